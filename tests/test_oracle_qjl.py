"""Pins for the oracle's QJL key format (oracle/qjl.py): the library Hadamard matrix, brute-force
sketches, hand-worked bit layouts, the exact residual identity, the estimator's unbiasedness over
sketch seeds (the property the QJL paper proves for its estimator) and the shrinkage it removes."""

import math

import numpy as np
import pytest
from scipy import linalg

from oracle import attention, codebook, qjl, quantize, rotation


@pytest.mark.parametrize("D", [8, 64, 128])
def test_sketch_is_library_hadamard_times_signs(D):
    sigma = rotation.signs(qjl.sketch_seed(5), D)
    np.testing.assert_array_equal(qjl.sketch_matrix(5, D), linalg.hadamard(D).astype(np.float64) * sigma)
    # an independent stream: not the rotation's signs
    assert not np.array_equal(sigma, rotation.signs(5, D))


def test_sketch_bits_by_brute_force(rng):
    """D = 8: with no MSE part (idx 0, stored norm 0) the residual is R x; bits by explicit sums."""
    D, seed = 8, 3
    x = rng.standard_normal((6, D)).astype(np.float16)
    bits, gamma, tie = qjl.encode(x, np.zeros((6, D), np.int64), np.zeros(6, np.float32),
                                  np.zeros(2, np.float32), seed)
    s = rotation.signs(seed, D)
    sig = rotation.signs(qjl.sketch_seed(seed), D)
    for r_ in range(6):
        xr = x[r_].astype(np.float64)
        v = [sum((-1) ** bin(i & j).count("1") * s[j] * xr[j] for j in range(D)) / math.sqrt(D) for i in range(D)]
        y = [sum((-1) ** bin(i & j).count("1") * sig[j] * v[j] for j in range(D)) for i in range(D)]
        assert [int(t >= 0) for t in y] == bits[r_].tolist()
        assert abs(float(gamma[r_]) - math.sqrt(sum(t * t for t in v))) <= 1e-6 * float(gamma[r_])
        assert not tie[r_].any()


def test_pack_layout_hand_worked():
    bits = np.zeros((1, 16), np.uint8)
    bits[0, [0, 9, 15]] = 1                    # byte 0 = 0b00000001, byte 1 = 0b10000010
    buf = qjl.pack(bits, np.array([1.5], np.float32))
    assert buf[0].tolist() == [0x01, 0x82, 0x00, 0x00, 0xC0, 0x3F]  # 1.5f = 0x3FC00000 LE
    b2, g2 = qjl.unpack(buf, 16)
    assert np.array_equal(b2, bits) and g2[0] == np.float32(1.5)


@pytest.mark.parametrize("mean", [False, True])
def test_residual_completes_the_row(mean, rng):
    """n_s R^T c[idx] + R^T r = x - mu 1 exactly (up to fp64 rounding), for plain and corrected norms."""
    D, bits = 128, 3
    cb = codebook.codebook(D, bits)
    x = (rng.standard_normal((20, D)) + (4.0 if mean else 0.0)).astype(np.float16)
    for corrected in (None, cb.centroids32):
        out = quantize.quantize_rows(x, cb.boundaries32, 7, corrected, mean)
        idx, n = out[0], out[1]
        mu = out[3] if mean else None
        r = qjl.residual(x, idx, n, cb.centroids32, 7, mu)
        R = rotation.rotation_matrix(7, D)
        back = quantize.dequantize_plain(idx, n, cb.centroids32, 7, mu) + r @ R
        np.testing.assert_allclose(back, x.astype(np.float64), rtol=0, atol=1e-9)


def test_zero_and_constant_rows_have_no_residual():
    D = 64
    cb = codebook.codebook(D, 2)
    for x, mean in ((np.zeros((1, D), np.float16), False), (np.full((1, D), 3.25, np.float16), True)):
        out = quantize.quantize_rows(x, cb.boundaries32, 0, mean=mean)
        bits, gamma, tie = qjl.encode(x, out[0], out[1], cb.centroids32, 0, out[3] if mean else None)
        assert gamma[0] == 0 and bits.all() and tie.all()
        assert np.all(qjl.residual_estimate(bits, gamma, 0) == 0)


def test_estimator_is_unbiased_over_sketches(rng):
    """E[q . k_tilde - q . k] = 0 over the layer seed (which draws the rotation and the sketch): the
    mean difference sits within 4 standard errors of 0, where a wrong factor (sqrt(2/pi) for
    sqrt(pi/2)), a flipped sign or a dropped residual norm is off by many."""
    D, bits_ = 128, 2
    cb = codebook.codebook(D, bits_)
    x = rng.standard_normal((1, D)).astype(np.float16)
    q = (x.astype(np.float64)[0] * 2 + rng.standard_normal(D) * 0.5)
    diffs, trues = [], []
    for seed in range(1500):
        idx, n, _ = quantize.quantize_rows(x, cb.boundaries32, seed)
        b, g, _ = qjl.encode(x, idx, n, cb.centroids32, seed)
        k_mse = quantize.dequantize_plain(idx, n, cb.centroids32, seed)[0]
        est = q @ k_mse + qjl.score_term(rotation.rotation_matrix(seed, D) @ q, b, g, seed)[0]
        diffs.append(est - q @ x.astype(np.float64)[0])
        trues.append(q @ (x.astype(np.float64)[0] - k_mse))
    diffs, trues = np.array(diffs), np.array(trues)
    se = diffs.std() / math.sqrt(len(diffs))
    assert abs(diffs.mean()) < 4 * se
    assert abs(trues.mean()) > 12 * se   # the residual's inner product is far from 0 on average


def test_qjl_removes_the_mse_shrinkage(rng):
    """Lloyd-Max reconstruction shrinks self inner products (E[x . x_hat] = E||x_hat||^2 < ||x||^2);
    the QJL-corrected key does not: mean(x . k_tilde) / mean(||x||^2) is 1 within 1 %."""
    D = 128
    cb = codebook.codebook(D, 2)
    x = rng.standard_normal((400, D)).astype(np.float16)
    idx, n, _ = quantize.quantize_rows(x, cb.boundaries32, 11)
    b, g, _ = qjl.encode(x, idx, n, cb.centroids32, 11)
    k_mse = quantize.dequantize_plain(idx, n, cb.centroids32, 11)
    k_q = k_mse + qjl.residual_estimate(b, g, 11)
    xx = x.astype(np.float64)
    ref = np.mean(np.sum(xx * xx, axis=1))
    assert np.mean(np.sum(xx * k_mse, axis=1)) / ref < 0.9
    assert abs(np.mean(np.sum(xx * k_q, axis=1)) / ref - 1) < 0.01


def test_dequant_and_score_routes_agree(rng):
    D, seed = 64, 9
    cb = codebook.codebook(D, 4)
    x = rng.standard_normal((30, D)).astype(np.float16)
    idx, n, _ = quantize.quantize_rows(x, cb.boundaries32, seed)
    b, g, _ = qjl.encode(x, idx, n, cb.centroids32, seed)
    q = rng.standard_normal(D)
    via_dequant = qjl.residual_estimate(b, g, seed) @ q
    via_scores = qjl.score_term(rotation.rotation_matrix(seed, D) @ q, b, g, seed)
    np.testing.assert_allclose(via_dequant, via_scores, rtol=0, atol=1e-12)


def test_slot_layout_and_readback(rng):
    D, H_kv, kb, vb = 128, 2, 3, 4
    assert quantize.slot_bytes(D, kb, vb, qjl=True) == quantize.slot_bytes(D, kb, vb) + D // 8 + 4
    assert quantize.slot_bytes(D, kb, vb, True, True) == 48 + 8 + 16 + 4 + 64 + 8
    ck, cv = codebook.codebook(D, kb), codebook.codebook(D, vb)
    k = rng.standard_normal((5, H_kv, D)).astype(np.float16)
    v = rng.standard_normal((5, H_kv, D)).astype(np.float16)
    for mean in (False, True):
        sb = quantize.slot_bytes(D, kb, vb, mean, True)
        pages = np.zeros(8 * H_kv * sb, np.uint8)
        slots = np.array([3, 0, -1, 7, 5])
        quantize.append_rows_fast(pages, k, v, slots, ck.boundaries32, cv.boundaries32, kb, vb, 2,
                                  mean=mean, qjl_centroids32=ck.centroids32)
        got = quantize.read_slots(pages, slots[slots >= 0], H_kv, D, kb, vb, None, mean, True)
        kq = quantize.quantize_rows(k[slots >= 0], ck.boundaries32, 2, None, mean)
        vq = quantize.quantize_rows(v[slots >= 0], cv.boundaries32, 2, None, mean)
        b, g, _ = qjl.encode(k[slots >= 0], kq[0], kq[1], ck.centroids32, 2, kq[3] if mean else None)
        assert np.array_equal(got[0], kq[0]) and np.array_equal(got[2], vq[0])
        assert np.array_equal(got[1], kq[1]) and np.array_equal(got[3], vq[1])
        assert np.array_equal(got[-2], b) and np.array_equal(got[-1], g)


@pytest.mark.parametrize("D, H_kv, G, kb, vb, L, ns, mean", [(64, 2, 2, 2, 4, 37, 0, False),
                                                             (128, 1, 4, 3, 2, 50, 4, True)])
def test_attention_routes_agree_with_qjl(D, H_kv, G, kb, vb, L, ns, mean, rng):
    ck, cv = codebook.codebook(D, kb), codebook.codebook(D, vb)
    nb = (L + 15) // 16
    bt = rng.permutation(nb + 2)[:nb]
    k = rng.standard_normal((L, H_kv, D)).astype(np.float16)
    v = rng.standard_normal((L, H_kv, D)).astype(np.float16)
    slots = bt[np.arange(L) // 16] * 16 + np.arange(L) % 16
    pages = np.zeros((nb + 2) * 16 * H_kv * quantize.slot_bytes(D, kb, vb, mean, True), np.uint8)
    quantize.append_rows_fast(pages, k, v, slots, ck.boundaries32, cv.boundaries32, kb, vb, 4,
                              mean=mean, qjl_centroids32=ck.centroids32)
    layer = dict(D=D, H_kv=H_kv, block_size=16, k_bits=kb, v_bits=vb, seed=4, mean=mean, qjl=True)
    q = rng.standard_normal((1, H_kv * G, D)).astype(np.float16)
    sk = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    args = (q, pages, bt[None], np.array([L]), layer, ck.centroids32, cv.centroids32, sk, sk, ns)
    np.testing.assert_allclose(attention.decode_attention(*args), attention.decode_attention_rotated(*args),
                               atol=1e-12, rtol=0)


@pytest.mark.parametrize("D, bits_, mean", [(64, 2, False), (128, 4, True), (128, 3, False)])
def test_dequantize_key_spec_matches_plain_route(D, bits_, mean, rng):
    """The library's bit-exact fp32 chain for QJL keys against the fp64 plain route n R^T c[idx] +
    sqrt(pi/2)/D gamma R^T S^T (2b - 1) (+ mu): within 3 roundings of the codes' and the residual's
    parts (plus one of the mean).  Planted slips (the sketch transform used for its transpose, a
    dropped sign vector, gamma left out) are far outside the bound."""
    seed = 6
    cb = codebook.codebook(D, bits_)
    x = (rng.standard_normal((40, D)) * 3.0 + (2.0 if mean else 0.0)).astype(np.float16)
    out = quantize.quantize_rows(x, cb.boundaries32, seed, None, mean)
    idx, n = out[0], out[1]
    mu = out[3] if mean else None
    b, g, _ = qjl.encode(x, idx, n, cb.centroids32, seed, mu)
    spec = qjl.dequantize_key_spec(idx, n, cb.centroids32, b, g, seed, mu).astype(np.float64)
    code = quantize.dequantize_plain(idx, n, cb.centroids32, seed)
    resid = qjl.residual_estimate(b, g, seed)
    plain = code + resid + (0.0 if mu is None else mu.astype(np.float64)[:, None])
    u = 2.0 ** -24
    bound = 3 * u * (np.abs(code) + np.abs(resid)) + (2 * u * np.abs(plain) if mean else 0.0)
    assert np.all(np.abs(spec - plain) <= bound)
    # the chain reads its own gamma and bits: a slip in either moves the result by far more
    R = rotation.rotation_matrix(seed, D)
    S = qjl.sketch_matrix(seed, D)
    z = 2.0 * b - 1.0
    wrong_t = (qjl.KAPPA_NUM / D) * g.astype(np.float64)[:, None] * ((z @ S.T) @ R)  # S for S^T
    assert np.max(np.abs(code + wrong_t + (plain - code - resid) - spec) - bound) > 0
    assert np.max(np.abs(code + (plain - code - resid) - spec) - bound) > 0      # gamma dropped
