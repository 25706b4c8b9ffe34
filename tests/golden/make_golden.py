"""Writes the stored regression values under tests/golden/ from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
Only oracle/ is imported; nothing here touches the GPU library.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import rotation  # noqa: E402


def main():
    s = rotation.signs(0, 64)
    with open(os.path.join(HERE, "signs_seed0_D64.txt"), "w") as f:
        f.write("# First 64 RHT signs for seed 0 (SplitMix64, '1' = -1), written by make_golden.py\n")
        f.write("".join("1" if v < 0 else "0" for v in s) + "\n")


if __name__ == "__main__":
    main()
