"""1-bit QJL residual on keys (oracle, fp64, dense).  Test infrastructure only.

Follows:
* tq-kv, "How It Works": step [5], SRHT QJL error correction, optional, O(d log d) (a
  subsampled-randomized-Hadamard sketch, as the rotation of step [3] is a randomized Hadamard).
* TorbuQuant docs, "Current Status": a QJL residual, used for vector and inner-product work.
* The TurboQuant paper (Zandieh et al., arXiv:2504.19874) and the QJL paper (Zandieh, Daliri, Han,
  arXiv:2406.03482), both in the TorbuQuant page's references: a key is quantized by the MSE
  quantizer, then the sign bits of a random projection of the residual and the residual's norm
  are stored, and an inner product with the key is estimated without bias by the MSE part plus
  sqrt(pi/2) / m * ||r|| * <S q, sign(S r)> (m rows of S; for rows with unit-variance entries,
  E[<s, q> sign(<s, r>)] = sqrt(2/pi) <q, r> / ||r||).

Readings taken where the pages are silent (each is also listed in the design notes)
----------------------------------------------------------------------------------
* Frame: everything happens in the rotated frame of the MSE quantizer.  v = R (x - mu 1) (mu = 0
  without mean removal) and the residual is r = v - n_s c[idx], with n_s the stored norm (plain,
  or corrected) and c the fp32 centroids; then n_s R^T c[idx] + R^T r = x - mu 1 exactly.
* Sketch: S = H_D diag(sigma), the SRHT with m = D rows (no subsampling): rows of +-1, so every
  row has unit-variance entries as the estimator needs.  sigma = rotation.signs(seed2, D) with
  seed2 = seed XOR QJL_SEED_XOR (a second, independent SplitMix64 stream of the layer's seed).
* Bits: b_i = 1 when (S r)_i >= 0, else 0; z_i = 2 b_i - 1.  gamma = fp32(||r||_2).  A zero
  residual gives gamma = 0 and every bit 1.  The residual is defined exactly; a kernel that forms
  r, ||r|| and S r in fp64 differs from it by about 1e-15 ||r||, so |(S r)_i| <= QJL_TIE * ||r||
  counts as a tie (either bit is accepted there), and so does a gamma whose fp64 value lies within
  QJL_TIE (relative) of an fp32 rounding midpoint (either neighbouring fp32 is accepted).
* Layout: the key region gains, after its norm (and mean), D/8 bytes of sketch bits, LSB-first
  (bit i in byte i // 8 at position i % 8), then gamma as little-endian fp32.  Values are not
  sketched.
* Estimate: the dequantized key gains sqrt(pi/2) / D * gamma * R^T S^T z, so that
  q . k_tilde = q . k_mse + sqrt(pi/2) / D * gamma * (S R q) . z, the QJL estimator with R q for q.
"""

from __future__ import annotations

import math

import numpy as np

from . import rotation

QJL_SEED_XOR = 0x514A4C5F534B4554  # "QJL_SKET"
QJL_TIE = 1e-12
KAPPA_NUM = math.sqrt(math.pi / 2.0)  # the estimator's factor is KAPPA_NUM / D


def sketch_seed(seed: int) -> int:
    """Seed of the sketch's sign vector sigma."""
    return (int(seed) ^ QJL_SEED_XOR) & ((1 << 64) - 1)


def sketch_matrix(seed: int, D: int) -> np.ndarray:
    """S = H_D diag(sigma), dense (entries +-1)."""
    return rotation.hadamard(D) * rotation.signs(sketch_seed(seed), D)[None, :]


def residual(x16: np.ndarray, idx: np.ndarray, n_store32, centroids32: np.ndarray, seed: int,
             mu32=None) -> np.ndarray:
    """r = R (x - mu 1) - n_s c[idx] in fp64, shaped like x16."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if mu32 is not None:
        x = x - np.asarray(mu32, np.float32).astype(np.float64)[..., None]
    D = x.shape[-1]
    v = x @ rotation.rotation_matrix(seed, D).T
    c = np.asarray(centroids32, np.float32).astype(np.float64)[np.asarray(idx)]
    return v - np.asarray(n_store32, np.float32).astype(np.float64)[..., None] * c


def encode(x16, idx, n_store32, centroids32, seed: int, mu32=None, with_gamma_tie: bool = False):
    """(bits uint8 in {0, 1} [..., D], gamma fp32 [...], tie bool [..., D]) of the key rows; with
    with_gamma_tie also the gamma tie mask [...] (see the module notes)."""
    r = residual(x16, idx, n_store32, centroids32, seed, mu32)
    D = r.shape[-1]
    y = r @ sketch_matrix(seed, D).T
    rn = np.sqrt(np.sum(r * r, axis=-1))
    bits = (y >= 0).astype(np.uint8)
    tie = np.abs(y) <= QJL_TIE * rn[..., None]
    if not with_gamma_tie:
        return bits, rn.astype(np.float32), tie
    g_tie = (rn * (1 - QJL_TIE)).astype(np.float32) != (rn * (1 + QJL_TIE)).astype(np.float32)
    return bits, rn.astype(np.float32), tie, g_tie


def pack(bits: np.ndarray, gamma32) -> np.ndarray:
    """bits [N, D] -> uint8 [N, D/8 + 4]: the sketch bytes LSB-first, then gamma (fp32 LE)."""
    bits = np.asarray(bits, dtype=np.uint8)
    N, D = bits.shape
    body = np.packbits(bits, axis=1, bitorder="little")
    g = np.asarray(gamma32, dtype="<f4").reshape(N, 1).view(np.uint8)
    return np.concatenate([body, g], axis=1)


def unpack(buf: np.ndarray, D: int):
    """Inverse of pack: uint8 [N, D/8 + 4] -> (bits uint8 [N, D], gamma fp32 [N])."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    N = buf.shape[0]
    bits = np.unpackbits(buf[:, :D // 8], axis=1, bitorder="little")[:, :D]
    gamma = np.ascontiguousarray(buf[:, D // 8:D // 8 + 4]).view("<f4").reshape(N).astype(np.float32)
    return bits, gamma


def residual_estimate(bits, gamma32, seed: int) -> np.ndarray:
    """The dequantized residual in the original frame: sqrt(pi/2) / D * gamma * R^T S^T z (fp64)."""
    z = 2.0 * np.asarray(bits, dtype=np.float64) - 1.0
    D = z.shape[-1]
    S = sketch_matrix(seed, D)
    R = rotation.rotation_matrix(seed, D)
    rot = z @ S                      # S^T z, row-wise
    return (KAPPA_NUM / D) * np.asarray(gamma32, np.float32).astype(np.float64)[..., None] * (rot @ R)


# The double nearest sqrt(pi/2) (0x1.40d931ff62706p+0).  math.sqrt(math.pi / 2) is one ulp below it
# because math.pi is below pi; the fp32 chain of dequantize_key_spec fixes this constant.
KAPPA_F64 = float.fromhex("0x1.40d931ff62706p+0")


def dequantize_key_spec(idx, norm32, centroids32, bits, gamma32, seed: int, mu32=None) -> np.ndarray:
    """Bit-exact fp32 dequantized key of the QJL key format (the chain the library states):
      z = H c[idx] exactly, g = fp32(n * fp32(1/sqrt(D))) (the codes' part, as quantize.dequantize_spec);
      t = H diag(sigma) H (2b - 1), exact integers (|t_i| <= D^2);
      gq = fp32(KAPPA_F64 / D * gamma * fp32(1/sqrt(D))), the product taken in fp64;
      x_i = s_i * fp32(fp32(fp32(z_i) * g) + fp32(fp32(t_i) * gq)), then fp32(x_i + mu).
    Since t = H S^T z_b and R^T = D^(-1/2) diag(s) H, this is n R^T c[idx] + sqrt(pi/2) / D * gamma
    * R^T S^T (2b - 1) (+ mu) with every rounding fixed; the pins hold it to the fp64 plain route."""
    from . import quantize as _q
    idx = np.asarray(idx)
    D = idx.shape[-1]
    chat = np.asarray(centroids32, dtype=np.float32)[idx]
    z32 = _q.exact_wht(chat).astype(np.float32)
    rD = np.float32(1.0 / math.sqrt(D))
    g = (np.asarray(norm32, dtype=np.float32) * rD).astype(np.float32)
    zb = 2.0 * np.asarray(bits, dtype=np.float64) - 1.0
    H = rotation.hadamard(D)
    sigma = rotation.signs(sketch_seed(seed), D)
    t = (zb @ H.T) * sigma
    t = t @ H.T
    assert np.all(t == np.round(t)) and np.max(np.abs(t), initial=0.0) <= D * D
    gq = ((KAPPA_F64 / D) * np.asarray(gamma32, np.float32).astype(np.float64)
          * np.float64(rD)).astype(np.float32)
    code = (z32 * g[..., None]).astype(np.float32)
    resid = (t.astype(np.float32) * gq[..., None]).astype(np.float32)
    s = rotation.signs(seed, D).astype(np.float32)
    x = (s * (code + resid).astype(np.float32)).astype(np.float32)
    if mu32 is not None:
        x = (x + np.asarray(mu32, np.float32)[..., None]).astype(np.float32)
    return x


def score_term(qrot: np.ndarray, bits, gamma32, seed: int) -> np.ndarray:
    """sqrt(pi/2) / D * gamma * (S q') . z for rotated queries q' = R q (fp64): the residual's part
    of q . k_tilde.  qrot [D]; bits [..., D]; gamma [...]."""
    z = 2.0 * np.asarray(bits, dtype=np.float64) - 1.0
    D = z.shape[-1]
    sq = sketch_matrix(seed, D) @ np.asarray(qrot, dtype=np.float64)
    return (KAPPA_NUM / D) * np.asarray(gamma32, np.float32).astype(np.float64) * (z @ sq)
