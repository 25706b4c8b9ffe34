"""Build the HIP library libtq.so in-tree for gfx950.

    python -m packed_decode_attention_amd.build            # or: python packed_decode_attention_amd/build.py

hipcc cross-compiles the device code for gfx950 without a GPU present.  Packed-fp32 VALU
instructions are disabled for all device code (-packed-fp32-ops).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtq.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
DEVICE_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-fno-strict-aliasing", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall"]

SOURCES = [
    ("tq_quantize.hip", "device"),
    ("tq_decode.hip", "device"),
    ("tq_api.cpp", "host"),
    ("tq_codebook.cpp", "host"),
]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, kind in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        path = os.path.join(CSRC, src)
        if kind == "device":
            _run([HIPCC, *DEVICE_FLAGS, "-c", path, "-o", obj])
        else:
            _run(["g++", *HOST_FLAGS, "-c", path, "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
