"""Randomized Hadamard rotation (oracle, fp64, dense).

Follows: tq-kv, "How It Works" step [3] (randomized Hadamard transform, O(d log d), to
decorrelate coordinates) and its "generate_signs(dim, seed)" call; TorbuQuant docs,
"Current Status" table (RHT rotation); turboquant-serve 0.1.2, "Architecture" (one fixed
rotation, seeded, shared by all requests).

Reading taken where the pages are silent
----------------------------------------
* Sign generator: SplitMix64 (Steele, Lea and Flood, OOPSLA 2014).  state starts at the seed;
  each draw adds the golden-ratio increment and applies the published finaliser; the sign of
  coordinate i is -1 when bit 63 of the i-th draw is set, +1 otherwise.  One sign vector per
  (seed, D), shared by every layer, head, and by K and V.
* R = D^(-1/2) H_D diag(s): sign flip first, then the Sylvester Hadamard matrix
  (H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]], so H[i, j] = (-1)^popcount(i & j)).
  R is orthogonal and R^T = D^(-1/2) diag(s) H_D.

The oracle forms R densely; it never uses a fast transform.
"""

from __future__ import annotations

import numpy as np

_MASK64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> list[int]:
    """First n outputs of SplitMix64 started at `seed` (Python integers, exact)."""
    state = seed & _MASK64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        z = z ^ (z >> 31)
        out.append(z)
    return out


def signs(seed: int, D: int) -> np.ndarray:
    """s in {-1, +1}^D: -1 where the top bit of the i-th SplitMix64 draw is set."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64(seed, D)], dtype=np.float64)


def hadamard(D: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_D (entries +-1, H_D @ H_D = D I), built by the doubling rule."""
    if D < 1 or (D & (D - 1)) != 0:
        raise ValueError("D must be a power of two")
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    return H


def rotation_matrix(seed: int, D: int) -> np.ndarray:
    """R = D^(-1/2) H_D diag(s)."""
    return hadamard(D) * signs(seed, D)[None, :] / np.sqrt(D)
