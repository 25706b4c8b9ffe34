"""Per-row quantize-on-append, TQ4 page slots and dequantization (oracle).

Follows:
* turboquant-serve 0.1.2, "Architecture": rotate, normalise to the unit sphere, Lloyd-Max
  encode, bit-pack, store uint8; decode = unpack, Lloyd-Max decode, restore magnitude,
  multiply by R^T.
* turboquant-pro 1.4.2, "How It Works": per-vector flow extract L2 norm -> normalise ->
  rotate -> Lloyd-Max quantise -> bit-pack, the norm kept alongside the bits.
* TorbuQuant docs, "TQ4 page tensor" figure: page tensor [num_blocks, block_size,
  num_kv_heads, slot_bytes] of uint8; block = slot // block_size, row = slot % block_size,
  page[block, row, kv_head, :]; the slot is a K region (packed K indices, then an fp32 norm)
  followed by a V region (packed V indices, then an fp32 norm); region bytes are
  ceil(D * bits / 8) + 4; the same norm-coded row packer serves K and V.

Readings taken where the pages are silent (each is also listed in the design notes)
----------------------------------------------------------------------------------
* Stored norm: the fp32 value of ||x||_2 of the fp16 row, computed as
  sq_i = fp32(x_i)^2 (exact), then a stride-halving fp32 tree (for h = D/2, D/4, ..., 1:
  sq_i <- sq_i + sq_{i+h} for i < h), then a correctly rounded fp32 square root.
* Rotated coordinate: u = R x / ||x|| (fp64 here).  Decision against the fp32 boundaries:
  idx_i = #{ j : t_j <= u_i } (a value exactly on a boundary goes up).  A coordinate within
  TIE_BAND of a boundary is reported as a tie; either neighbouring index is accepted there.
* Zero row (norm 0): every index is L/2 (u = 0 sits on the middle boundary, which is exactly
  0, and goes up) and the norm bytes are zero.
* Packing: LSB-first bitstream; index i occupies bits [i*b, (i+1)*b) of the region, byte k
  holds bits 8k..8k+7.  The norm follows as little-endian IEEE binary32.  Bytes between
  slot_bytes and a larger slot stride are zero.
* Dequantized row (bit-exact route): c_hat_i = c[idx_i] (fp32); z = H c_hat exactly (fp64 is
  exact here, asserted); g = fp32(n * fp32(1/sqrt(D))); x_hat_i = s_i * fp32(fp32(z_i) * g).
* Per-token mean removal (format flag; tq-kv, "How It Works": the quantiser's per-token mean
  removal stage, and the mean in its output record): mu = fp32(tree(fp32(x_i))) / D (the
  stride-halving fp32 tree of the row's values; division by the power of two D is exact); the
  row is centred, d_i = fp32(x_i - mu); the stored norm is n = fp32 sqrt(tree(fp32(d_i^2))); the
  rotated coordinate is u = R (x - mu 1) / ||x - mu 1|| (fp64); the region gains mu as a second
  fp32 after the norm; the dequantized row is fp32(x_hat_i + mu) (plain route: n R^T c + mu 1).
  A constant row has d = 0: it stores norm 0, indices L/2 and mu = its value, and dequantizes
  exactly.
* Norm correction (format flag; tq-kv, "How It Works": "Lloyd-Max codebook + norm correction",
  output "packed indices + corrected norm"): the stored norm is n' = n / ||c_hat||_2, so the
  dequantized row n' R^T c_hat keeps the input row's L2 norm.  ||c_hat||^2 is the stride-halving
  fp32 tree (as for the norm, over rotated coordinates) of fp32(c_hat_i^2), then a correctly
  rounded fp32 square root and a correctly rounded fp32 division; a zero norm stays 0.
"""

from __future__ import annotations

import math

import numpy as np

from . import rotation

TIE_BAND = 1e-6


# --------------------------------------------------------------------------------------------
# Sizes.
# --------------------------------------------------------------------------------------------
def region_bytes(D: int, bits: int, mean: bool = False) -> int:
    """ceil(D * bits / 8) packed index bytes + 4 bytes of fp32 norm (TQ4 page tensor figure), + 4
    bytes of fp32 mean with mean removal."""
    return (D * bits + 7) // 8 + 4 + (4 if mean else 0)


def qjl_bytes(D: int, qjl: bool) -> int:
    """QJL key format: D/8 bytes of residual sketch bits + 4 bytes of fp32 residual norm."""
    return D // 8 + 4 if qjl else 0


def key_region_bytes(D: int, k_bits: int, mean: bool = False, qjl: bool = False) -> int:
    """K region: codes, norm (and mean), then the QJL sketch and residual norm."""
    return region_bytes(D, k_bits, mean) + qjl_bytes(D, qjl)


def slot_bytes(D: int, k_bits: int, v_bits: int, mean: bool = False, qjl: bool = False) -> int:
    """K region + V region (TQ4 page tensor figure)."""
    return key_region_bytes(D, k_bits, mean, qjl) + region_bytes(D, v_bits, mean)


# --------------------------------------------------------------------------------------------
# Norm, rotation, index decision.
# --------------------------------------------------------------------------------------------
def norm_fp32(x16: np.ndarray) -> np.ndarray:
    """Stored fp32 norm of each fp16 row: exact squares, stride-halving fp32 tree, fp32 sqrt."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    return np.sqrt(_tree_sum32((x * x).astype(np.float32))).astype(np.float32)


def row_mean(x16: np.ndarray) -> np.ndarray:
    """Mean-removal format: mu = fp32(stride-halving fp32 tree of the fp16 values) / D."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    return (_tree_sum32(x) / np.float32(x.shape[-1])).astype(np.float32)


def centered_norm(x16: np.ndarray, mu32: np.ndarray) -> np.ndarray:
    """Mean-removal format: d_i = fp32(x_i - mu), n = fp32 sqrt(tree(fp32(d_i^2)))."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    d = (x - np.asarray(mu32, np.float32)[..., None]).astype(np.float32)
    return np.sqrt(_tree_sum32((d * d).astype(np.float32))).astype(np.float32)


def rotated_unit(x16: np.ndarray, seed: int, mu32=None) -> np.ndarray:
    """u = R x / ||x|| in fp64 (rows of zeros give u = 0); with mu32, u = R (x - mu) / ||x - mu||."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    if mu32 is not None:
        x = x - np.asarray(mu32, np.float32).astype(np.float64)[..., None]
    R = rotation.rotation_matrix(seed, x.shape[-1])
    y = x @ R.T
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    with np.errstate(invalid="ignore", divide="ignore"):
        u = np.where(n > 0, y / np.where(n > 0, n, 1.0), 0.0)
    return u


def indices_for(u: np.ndarray, boundaries32: np.ndarray):
    """idx = #{ j : t_j <= u } against the fp32 boundaries; also the tie mask."""
    t = np.asarray(boundaries32, dtype=np.float32).astype(np.float64)
    idx = np.zeros(u.shape, dtype=np.int64)
    tie = np.zeros(u.shape, dtype=bool)
    for tj in t:
        idx += (tj <= u)
        tie |= np.abs(u - tj) <= TIE_BAND
    return idx, tie


def _tree_sum32(sq32: np.ndarray) -> np.ndarray:
    """Stride-halving fp32 tree over the last axis: pairs (i, i + D/2) first, then D/4, ..."""
    sq = np.asarray(sq32, dtype=np.float32)
    h = sq.shape[-1] // 2
    while h >= 1:
        sq = (sq[..., :h] + sq[..., h:2 * h]).astype(np.float32)
        h //= 2
    return sq[..., 0]


def corrected_norm(n32: np.ndarray, idx: np.ndarray, centroids32: np.ndarray) -> np.ndarray:
    """Norm correction: n' = fp32(n / fp32(sqrt(tree(fp32(c[idx]^2))))), 0 where n == 0."""
    c = np.asarray(centroids32, dtype=np.float32)[np.asarray(idx)]
    r = np.sqrt(_tree_sum32((c * c).astype(np.float32))).astype(np.float32)
    n = np.asarray(n32, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (n / r).astype(np.float32)
    return np.where(n > 0, q, np.float32(0)).astype(np.float32)


def quantize_rows(x16: np.ndarray, boundaries32: np.ndarray, seed: int, centroids32=None,
                  mean: bool = False):
    """Quantize fp16 rows [..., D]: returns (idx int64 [..., D], norm fp32 [...], tie bool [..., D]),
    and with mean removal also mu fp32 [...] as a fourth value.  With centroids32 the stored norm
    is the corrected one (norm-correction format)."""
    mu = row_mean(x16) if mean else None
    u = rotated_unit(x16, seed, mu)
    idx, tie = indices_for(u, boundaries32)
    n = centered_norm(x16, mu) if mean else norm_fp32(x16)
    if centroids32 is not None:
        n = corrected_norm(n, idx, centroids32)
    return (idx, n, tie, mu) if mean else (idx, n, tie)


# --------------------------------------------------------------------------------------------
# Bit packing.
# --------------------------------------------------------------------------------------------
def pack_region(idx: np.ndarray, norm: np.float32, bits: int) -> bytes:
    """Pack one row: LSB-first bitstream of the D indices, then the fp32 norm little-endian."""
    D = len(idx)
    nbytes = (D * bits + 7) // 8
    acc = 0
    for i, v in enumerate(idx):
        v = int(v)
        assert 0 <= v < (1 << bits)
        acc |= v << (i * bits)
    body = acc.to_bytes(nbytes, "little")
    return body + np.asarray(norm, dtype="<f4").tobytes()


def unpack_region(buf: bytes, D: int, bits: int):
    """Inverse of pack_region: (idx list, fp32 norm)."""
    nbytes = (D * bits + 7) // 8
    acc = int.from_bytes(bytes(buf[:nbytes]), "little")
    mask = (1 << bits) - 1
    idx = np.array([(acc >> (i * bits)) & mask for i in range(D)], dtype=np.int64)
    norm = np.frombuffer(bytes(buf[nbytes:nbytes + 4]), dtype="<f4")[0]
    return idx, np.float32(norm)


# --------------------------------------------------------------------------------------------
# Page slots.
# --------------------------------------------------------------------------------------------
def slot_offset(slot: int, h: int, num_kv_heads: int, slot_stride: int) -> int:
    """Byte offset of page[slot // block_size, slot % block_size, h, :] in the flat page tensor."""
    return (slot * num_kv_heads + h) * slot_stride


def append_rows(pages: np.ndarray, k16: np.ndarray, v16: np.ndarray, slot_mapping: np.ndarray,
                k_boundaries32, v_boundaries32, k_bits: int, v_bits: int, seed: int,
                slot_stride: int | None = None, k_centroids32=None, v_centroids32=None):
    """Quantize-on-append: write the K and V regions of every (token, kv head) into its slot.

    pages: flat uint8 array of num_blocks * block_size * H_kv * slot_stride bytes (modified).
    k16, v16: [n_tok, H_kv, D] fp16.  slot_mapping: [n_tok]; a negative slot skips the token.
    Returns the tie masks (k_tie, v_tie), shaped [n_tok, H_kv, D].
    k_centroids32 / v_centroids32 (both or neither): store corrected norms.
    """
    n_tok, H_kv, D = k16.shape
    sb = slot_bytes(D, k_bits, v_bits)
    stride = sb if slot_stride is None else slot_stride
    k_idx, k_n, k_tie = quantize_rows(k16, k_boundaries32, seed, k_centroids32)
    v_idx, v_n, v_tie = quantize_rows(v16, v_boundaries32, seed, v_centroids32)
    for t in range(n_tok):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        for h in range(H_kv):
            off = slot_offset(s, h, H_kv, stride)
            row = pack_region(k_idx[t, h], k_n[t, h], k_bits) + pack_region(v_idx[t, h], v_n[t, h], v_bits)
            row = row + bytes(stride - sb)
            pages[off:off + stride] = np.frombuffer(row, dtype=np.uint8)
    return k_tie, v_tie


def read_slot(pages: np.ndarray, slot: int, h: int, H_kv: int, D: int, k_bits: int, v_bits: int,
              slot_stride: int | None = None):
    """Unpack one slot: ((k_idx, k_norm), (v_idx, v_norm))."""
    stride = slot_bytes(D, k_bits, v_bits) if slot_stride is None else slot_stride
    off = slot_offset(slot, h, H_kv, stride)
    kr = region_bytes(D, k_bits)
    buf = bytes(pages[off:off + stride])
    return unpack_region(buf[:kr], D, k_bits), unpack_region(buf[kr:], D, v_bits)


# --------------------------------------------------------------------------------------------
# Dequantization.
# --------------------------------------------------------------------------------------------
def exact_wht(chat32: np.ndarray) -> np.ndarray:
    """z = H c_hat for fp32 inputs, in fp64, with an integer cross-check that it is exact."""
    c = np.asarray(chat32, dtype=np.float32).astype(np.float64)
    D = c.shape[-1]
    H = rotation.hadamard(D)
    z = c @ H.T
    # exactness: every fp32 value is an integer multiple of 2^e_min; do the same sum in int64.
    nz = c[c != 0]
    if nz.size:
        _, e = np.frexp(np.abs(nz))
        e_min = int(e.min()) - 24
        scaled = np.ldexp(c, -e_min)
        assert np.all(scaled == np.round(scaled))
        zi = scaled.astype(np.int64) @ H.T.astype(np.int64)
        assert np.max(np.abs(zi)) < 2 ** 53
        assert np.array_equal(np.ldexp(zi.astype(np.float64), e_min), z), "fp64 WHT not exact"
    return z


def dequantize_spec(idx: np.ndarray, norm32, centroids32: np.ndarray, seed: int, mu32=None) -> np.ndarray:
    """Bit-exact fp32 reconstruction: x_hat_i = s_i * fp32(fp32(z_i) * fp32(n * fp32(1/sqrt(D)))),
    then fp32(x_hat_i + mu) with mean removal."""
    idx = np.asarray(idx)
    D = idx.shape[-1]
    chat = np.asarray(centroids32, dtype=np.float32)[idx]
    z32 = exact_wht(chat).astype(np.float32)
    rD = np.float32(1.0 / math.sqrt(D))
    g = (np.asarray(norm32, dtype=np.float32) * rD).astype(np.float32)
    s = rotation.signs(seed, D).astype(np.float32)
    x = (s * (z32 * g[..., None]).astype(np.float32)).astype(np.float32)
    if mu32 is not None:
        x = (x + np.asarray(mu32, np.float32)[..., None]).astype(np.float32)
    return x


def dequantize_plain(idx: np.ndarray, norm32, centroids32: np.ndarray, seed: int, mu32=None) -> np.ndarray:
    """x_hat = n R^T c_hat (+ mu 1 with mean removal), in fp64 (the plain definition)."""
    idx = np.asarray(idx)
    D = idx.shape[-1]
    chat = np.asarray(centroids32, dtype=np.float32).astype(np.float64)[idx]
    R = rotation.rotation_matrix(seed, D)
    x = np.asarray(norm32, dtype=np.float64)[..., None] * (chat @ R)
    if mu32 is not None:
        x = x + np.asarray(mu32, np.float32).astype(np.float64)[..., None]
    return x


# --------------------------------------------------------------------------------------------
# Vectorised forms of the packer (same bitstream; pinned against the per-row forms above).
# --------------------------------------------------------------------------------------------
def pack_regions(idx: np.ndarray, norms: np.ndarray, bits: int, means=None) -> np.ndarray:
    """Pack many rows at once: idx [N, D] -> uint8 [N, region_bytes(D, bits)] (the mean, when
    given, follows the norm)."""
    idx = np.asarray(idx, dtype=np.int64)
    N, D = idx.shape
    bitplanes = ((idx[:, :, None] >> np.arange(bits)[None, None, :]) & 1).astype(np.uint8)
    body = np.packbits(bitplanes.reshape(N, D * bits), axis=1, bitorder="little")
    parts = [body, np.asarray(norms, dtype="<f4").reshape(N, 1).view(np.uint8)]
    if means is not None:
        parts.append(np.asarray(means, dtype="<f4").reshape(N, 1).view(np.uint8))
    return np.concatenate(parts, axis=1)


def unpack_means(buf: np.ndarray, D: int, bits: int) -> np.ndarray:
    """The fp32 means of mean-removal regions uint8 [N, region_bytes(D, bits, True)]."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    nbytes = (D * bits + 7) // 8
    return np.ascontiguousarray(buf[:, nbytes + 4:nbytes + 8]).view("<f4").reshape(-1).astype(np.float32)


def unpack_regions(buf: np.ndarray, D: int, bits: int):
    """Inverse of pack_regions: uint8 [N, region_bytes] -> (idx int64 [N, D], norms fp32 [N])."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    N = buf.shape[0]
    nbytes = (D * bits + 7) // 8
    planes = np.unpackbits(buf[:, :nbytes], axis=1, bitorder="little")[:, :D * bits]
    planes = planes.reshape(N, D, bits).astype(np.int64)
    idx = np.sum(planes << np.arange(bits)[None, None, :], axis=2)
    norms = np.ascontiguousarray(buf[:, nbytes:nbytes + 4]).view("<f4").reshape(N).astype(np.float32)
    return idx, norms


def append_rows_fast(pages: np.ndarray, k16, v16, slot_mapping, k_boundaries32, v_boundaries32,
                     k_bits: int, v_bits: int, seed: int, slot_stride: int | None = None,
                     k_centroids32=None, v_centroids32=None, mean: bool = False, qjl_centroids32=None):
    """append_rows() with the vectorised packer (same bytes; used for larger test cases); mean:
    the mean-removal format; qjl_centroids32 (the K centroids): the QJL key format, and the sketch
    tie masks (bits [n_tok, H_kv, D], gamma [n_tok, H_kv]) are returned third, as a pair."""
    from . import qjl as _qjl
    qjl = qjl_centroids32 is not None
    n_tok, H_kv, D = k16.shape
    sb = slot_bytes(D, k_bits, v_bits, mean, qjl)
    stride = sb if slot_stride is None else slot_stride
    kq = quantize_rows(k16, k_boundaries32, seed, k_centroids32, mean)
    vq = quantize_rows(v16, v_boundaries32, seed, v_centroids32, mean)
    (k_idx, k_n, k_tie), (v_idx, v_n, v_tie) = kq[:3], vq[:3]
    k_mu = kq[3].reshape(-1) if mean else None
    v_mu = vq[3].reshape(-1) if mean else None
    rows = np.zeros((n_tok, H_kv, stride), dtype=np.uint8)
    kr = region_bytes(D, k_bits, mean)
    kq_end = key_region_bytes(D, k_bits, mean, qjl)
    rows[:, :, :kr] = pack_regions(k_idx.reshape(-1, D), k_n.reshape(-1), k_bits, k_mu).reshape(n_tok, H_kv, kr)
    q_tie = None
    if qjl:
        bits, gamma, b_tie, g_tie = _qjl.encode(k16, k_idx, k_n, qjl_centroids32, seed,
                                                kq[3] if mean else None, with_gamma_tie=True)
        q_tie = (b_tie, g_tie)
        rows[:, :, kr:kq_end] = _qjl.pack(bits.reshape(-1, D), gamma.reshape(-1)).reshape(n_tok, H_kv, kq_end - kr)
    rows[:, :, kq_end:sb] = pack_regions(v_idx.reshape(-1, D), v_n.reshape(-1), v_bits, v_mu).reshape(n_tok, H_kv, sb - kq_end)
    view = pages.reshape(-1, H_kv, stride)
    sm = np.asarray(slot_mapping, dtype=np.int64)
    keep = sm >= 0
    view[sm[keep]] = rows[keep]
    return (k_tie, v_tie, q_tie) if qjl else (k_tie, v_tie)


def read_slots(pages: np.ndarray, slots: np.ndarray, H_kv: int, D: int, k_bits: int, v_bits: int,
               slot_stride: int | None = None, mean: bool = False, qjl: bool = False):
    """Unpack many slots: returns (k_idx, k_n, v_idx, v_n) shaped [n, H_kv, D] / [n, H_kv],
    (k_mu, v_mu) [n, H_kv] after them for the mean-removal format, then (sketch bits [n, H_kv, D],
    gamma [n, H_kv]) for the QJL key format."""
    from . import qjl as _qjl
    sb = slot_bytes(D, k_bits, v_bits, mean, qjl)
    stride = sb if slot_stride is None else slot_stride
    view = pages.reshape(-1, H_kv, stride)
    rows = view[np.asarray(slots, dtype=np.int64)]            # [n, H_kv, stride]
    n = rows.shape[0]
    kr = region_bytes(D, k_bits, mean)
    kq_end = key_region_bytes(D, k_bits, mean, qjl)
    kbuf = rows[:, :, :kr].reshape(n * H_kv, kr)
    vbuf = rows[:, :, kq_end:sb].reshape(n * H_kv, sb - kq_end)
    k_idx, k_n = unpack_regions(kbuf, D, k_bits)
    v_idx, v_n = unpack_regions(vbuf, D, v_bits)
    out = (k_idx.reshape(n, H_kv, D), k_n.reshape(n, H_kv), v_idx.reshape(n, H_kv, D), v_n.reshape(n, H_kv))
    if mean:
        out += (unpack_means(kbuf, D, k_bits).reshape(n, H_kv), unpack_means(vbuf, D, v_bits).reshape(n, H_kv))
    if qjl:
        bits, gamma = _qjl.unpack(rows[:, :, kr:kq_end].reshape(n * H_kv, kq_end - kr), D)
        out += (bits.reshape(n, H_kv, D), gamma.reshape(n, H_kv))
    return out
