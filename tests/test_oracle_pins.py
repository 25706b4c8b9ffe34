"""Pins for the CPU oracle: closed forms, textbook values, the pages' printed byte counts,
hand-worked fixtures and brute force.  None of these re-types the oracle's own formulas."""

import math
import os

import numpy as np
import pytest
from scipy import integrate, special

from oracle import attention, codebook, quantize, rotation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ============================================================================================
# Codebook
# ============================================================================================
def _sphere_pdf(D):
    """Textbook density of one coordinate of a uniform point on S^{D-1} (written out here)."""
    logC = math.lgamma(D / 2) - math.lgamma((D - 1) / 2) - 0.5 * math.log(math.pi)
    return lambda x: math.exp(logC + (D - 3) / 2 * math.log1p(-x * x)) if abs(x) < 1 else 0.0


@pytest.mark.parametrize("D, printed", [(64, 0.1001259082), (128, 0.0706615727), (256, None)])
def test_one_bit_beta_closed_form(D, printed):
    # 1 level per half: c = E[X | X > 0] = Gamma(D/2) / (sqrt(pi) Gamma((D+1)/2))
    want = math.exp(math.lgamma(D / 2) - math.lgamma((D + 1) / 2)) / math.sqrt(math.pi)
    cb = codebook.lloyd_max(D, 1, "beta")
    assert cb.boundaries[0] == 0.0
    assert abs(cb.centroids[1] - want) < 1e-13 and cb.centroids[0] == -cb.centroids[1]
    if printed is not None:
        assert abs(cb.centroids[1] - printed) < 1e-10


@pytest.mark.parametrize("D", [64, 128])
def test_one_bit_gaussian_closed_form(D):
    cb = codebook.lloyd_max(D, 1, "gaussian")
    assert abs(cb.centroids[1] - math.sqrt(2 / (math.pi * D))) < 1e-13
    assert abs(D * cb.mse - (1 - 2 / math.pi)) < 1e-12


# Max (1960) optimum quantizer for a unit Gaussian: outputs, thresholds and mean square error.
MAX_1960 = {
    2: dict(c=[0.4528, 1.510], t=[0.0, 0.9816], mse=0.1175),
    3: dict(c=[0.2451, 0.7560, 1.344, 2.152], t=[0.0, 0.5006, 1.050, 1.748], mse=0.03455),
    4: dict(c=[0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733],
            t=[0.0, 0.2582, 0.5224, 0.7996, 1.099, 1.437, 1.844, 2.401], mse=0.009497),
}


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_gaussian_matches_max_1960(bits):
    D = 128
    cb = codebook.lloyd_max(D, bits, "gaussian")
    s = math.sqrt(D)
    L = 1 << bits
    upper_c = cb.centroids[L // 2:] * s
    upper_t = cb.boundaries[L // 2 - 1:] * s
    ref = MAX_1960[bits]
    np.testing.assert_allclose(upper_c, ref["c"], atol=2e-3)
    np.testing.assert_allclose(upper_t, ref["t"], atol=2e-3)
    assert abs(D * cb.mse - ref["mse"]) < 2e-5


@pytest.mark.parametrize("family", ["beta", "gaussian"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_codebook_conditions(family, D, bits):
    cb = codebook.codebook(D, bits, family)
    c, t = cb.centroids, cb.boundaries
    L = 1 << bits
    assert c.shape == (L,) and t.shape == (L - 1,)
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])                     # exact symmetry
    assert t[L // 2 - 1] == 0.0                            # middle boundary exactly zero
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-16)
    assert cb.residual <= 1e-12
    # fp32 arrays: independently rounded, still strictly interleaved
    c32, t32 = cb.centroids32, cb.boundaries32
    assert c32.dtype == np.float32 and np.all(c32[:-1] < t32) and np.all(t32 < c32[1:])


@pytest.mark.parametrize("D, bits", [(64, 2), (128, 3), (128, 4), (64, 8)])
def test_beta_centroids_and_mse_by_quadrature(D, bits):
    """Centroid condition and MSE re-derived by direct numerical integration of the pdf."""
    cb = codebook.codebook(D, bits, "beta")
    pdf = _sphere_pdf(D)
    edges = np.concatenate(([-1.0], cb.boundaries, [1.0]))
    mse = 0.0
    L = 1 << bits
    check = range(L) if L <= 16 else list(range(0, L, 17)) + [L // 2, L - 1]
    for j in range(L):
        a, b = edges[j], edges[j + 1]
        p = integrate.quad(pdf, a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        e2 = integrate.quad(lambda x: (x - cb.centroids[j]) ** 2 * pdf(x), a, b,
                            epsabs=1e-17, epsrel=1e-12, limit=200)[0]
        mse += e2
        if j in check:
            assert abs(m1 / p - cb.centroids[j]) < 1e-10 * max(1.0, abs(cb.centroids[j])) + 1e-12
    assert abs(mse - cb.mse) < 1e-10 * 1 / D + 1e-14


def test_beta_cdf_matches_quadrature():
    for D in (64, 128):
        pdf = _sphere_pdf(D)
        dist = codebook.density(D, "beta")
        for x in (-0.5, -0.1, 0.0, 0.03, 0.2, 0.4):
            q = integrate.quad(pdf, -1.0, x, epsabs=1e-15, epsrel=1e-13)[0]
            assert abs(float(dist.cdf(x)) - q) < 1e-12


def test_mse_falls_with_bits_and_approaches_gaussian():
    for family in ("beta", "gaussian"):
        for D in (64, 128):
            m = [codebook.codebook(D, b, family).mse for b in (1, 2, 3, 4, 8)]
            assert all(m[i] > m[i + 1] for i in range(len(m) - 1))
    # D * MSE of the sphere law increases towards the Gaussian limit as D grows
    printed_b1 = {64: 0.35839, 128: 0.36089, 256: 0.36214}
    for D, v in printed_b1.items():
        assert abs(D * codebook.codebook(D, 1, "beta").mse - v) < 1e-5
    for bits in (1, 2, 3, 4):
        seq = [D * codebook.codebook(D, bits, "beta").mse for D in (64, 128, 256, 1024)]
        g = 128 * codebook.codebook(128, bits, "gaussian").mse
        assert all(seq[i] < seq[i + 1] for i in range(3)) and seq[-1] < g
        assert g - seq[-1] < 0.01 * g


def test_lloyd_from_a_bad_start_converges_to_same_point():
    """The fixed point is unique (log-concave density): plain Lloyd sweeps from a uniform start agree."""
    D, bits = 128, 3
    cb = codebook.codebook(D, bits, "beta")
    dist = codebook.density(D, "beta")
    c = np.linspace(-0.3, 0.3, 1 << bits)
    for _ in range(5000):
        t = 0.5 * (c[:-1] + c[1:])
        c_new, _ = codebook.centroids_for(dist, t)
        if np.max(np.abs(c_new - c)) < 1e-15:
            break
        c = c_new
    np.testing.assert_allclose(c, cb.centroids, atol=1e-12)


# ============================================================================================
# Rotation
# ============================================================================================
def test_splitmix64_published_vectors():
    # SplitMix64 reference outputs (seed 1234567 is the usual published test vector).
    assert rotation.splitmix64(1234567, 5) == [6457827717110365317, 3203168211198807973,
                                               9817491932198370423, 4593380528125082431,
                                               16408922859458223821]
    assert rotation.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_signs_seed0_frozen():
    s = rotation.signs(0, 64)
    bits = "".join("1" if v < 0 else "0" for v in s)
    with open(os.path.join(GOLDEN, "signs_seed0_D64.txt")) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    assert bits == lines[0]
    assert rotation.signs(0, 128)[:64].tolist() == s.tolist()   # prefix property of the stream


@pytest.mark.parametrize("D", [1, 2, 8, 64, 128])
def test_hadamard(D):
    H = rotation.hadamard(D)
    idx = np.arange(D)
    pop = np.vectorize(lambda v: bin(v).count("1"))(idx[:, None] & idx[None, :])
    assert np.array_equal(H, (-1.0) ** pop)
    assert np.array_equal(H @ H, D * np.eye(D))


@pytest.mark.parametrize("D", [64, 128])
def test_rotation_orthogonal_and_matches_butterflies(D, rng):
    R = rotation.rotation_matrix(0, D)
    np.testing.assert_allclose(R @ R.T, np.eye(D), atol=1e-14)
    x = rng.standard_normal((5, D))
    np.testing.assert_allclose(np.linalg.norm(x @ R.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # fast route written independently: flip signs, then in-place butterflies, then scale
    y = x * rotation.signs(0, D)
    h = 1
    while h < D:
        y = y.reshape(5, D // (2 * h), 2, h)
        y = np.stack([y[:, :, 0] + y[:, :, 1], y[:, :, 0] - y[:, :, 1]], axis=2).reshape(5, D)
        h *= 2
    np.testing.assert_allclose(y / np.sqrt(D), x @ R.T, atol=1e-12)


# ============================================================================================
# Quantize, pack, slots, dequantize
# ============================================================================================
def _load_pack_examples():
    out = []
    with open(os.path.join(GOLDEN, "pack_examples.txt")) as f:
        for ln in f:
            if not ln.strip() or ln.startswith("#"):
                continue
            b, idx, n, hx = [p.strip() for p in ln.split("|")]
            out.append((int(b), [int(v) for v in idx.split(",")], float(n), bytes.fromhex(hx)))
    return out


@pytest.mark.parametrize("case", _load_pack_examples())
def test_pack_golden(case):
    bits, idx, n, want = case
    got = quantize.pack_region(np.array(idx), np.float32(n), bits)
    assert got == want
    back, nb = quantize.unpack_region(got, len(idx), bits)
    assert back.tolist() == idx and nb == np.float32(n)
    vec = quantize.pack_regions(np.array([idx]), np.array([n], np.float32), bits)
    assert bytes(vec[0]) == want


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_roundtrip(D, bits, rng):
    idx = rng.integers(0, 1 << bits, size=(7, D))
    n = rng.random(7).astype(np.float32)
    vec = quantize.pack_regions(idx, n, bits)
    assert vec.shape == (7, quantize.region_bytes(D, bits))
    for r in range(7):
        assert bytes(vec[r]) == quantize.pack_region(idx[r], n[r], bits)
    i2, n2 = quantize.unpack_regions(vec, D, bits)
    assert np.array_equal(i2, idx) and np.array_equal(n2, n)


def test_slot_bytes_formula_and_printed_counts():
    sb = quantize.slot_bytes
    # per-config slots: K4/V4 D128, q8/q8 D64, K8/V4, K8/V8, K3/V2
    assert [sb(128, 4, 4), sb(64, 8, 8), sb(128, 8, 4), sb(128, 8, 8), sb(128, 3, 2)] == [136, 136, 200, 264, 88]
    rb = quantize.region_bytes
    # turboquant-pro 1.4.2, compression table on random Gaussian KV, head_dim 256 vs fp16:
    # 2/3/4 bits -> 7.5x / 5.1x / 3.9x
    assert [round(512 / rb(256, b), 1) for b in (2, 3, 4)] == [7.5, 5.1, 3.9]
    # core compressor at dim 1024 vs fp32: 15.8x (2-bit), 10.6x (3-bit), 7.9x (4-bit)
    assert [round(4096 / rb(1024, b), 1) for b in (2, 3, 4)] == [15.8, 10.6, 7.9]
    # pgvector example: 1024-dim 3-bit = 388 bytes; PCA-Matryoshka 384-dim 3-bit ~ 148 bytes
    assert rb(1024, 3) == 388 and rb(384, 3) == 148
    # "8 x 3-bit = 3 bytes"
    assert (8 * 3 + 7) // 8 == rb(8, 3) - 4 == 3


def test_norm_tree():
    x = np.zeros(128, np.float16)
    x[0], x[1] = 3, 4
    assert quantize.norm_fp32(x) == np.float32(5.0)
    rng = np.random.default_rng(7)
    for scale in (1e-3, 1.0, 30.0, 2000.0):
        X = (rng.standard_normal((500, 128)) * scale).astype(np.float16)
        got = quantize.norm_fp32(X).astype(np.float64)
        exact = np.sqrt(np.sum(X.astype(np.float64) ** 2, axis=1))
        ulp = np.spacing(exact.astype(np.float32)).astype(np.float64)
        # 7 levels of fp32 rounding (relative <= 7 * 2^-24 on the sum, halved by the root) plus
        # the root's own half ulp: at most ~2.3 ulp; one wrong level or a dropped term is far off.
        assert np.all(np.abs(got - exact) <= 2.5 * ulp)
    assert quantize.norm_fp32(np.zeros((3, 64), np.float16)).tolist() == [0.0, 0.0, 0.0]


def test_norm_tree_by_brute_force():
    # One row's stride-halving fp32 tree written out element by element: pairs (i, i + D/2) first,
    # then D/4, ..., every sum rounded to fp32, then a correctly rounded fp32 square root.  The row
    # is drawn so that summing adjacent pairs first, or accumulating in fp64 with one final
    # rounding, gives a different fp32 value: either mistake in norm_fp32 fails here.
    D = 32
    rng = np.random.default_rng(2024)
    for _ in range(1000):
        x = (rng.standard_normal(D) * np.exp(2.0 * rng.standard_normal(D))).astype(np.float16)
        sq = [np.float32(np.float32(v) * np.float32(v)) for v in x]
        vals = list(sq)
        h = D // 2
        while h >= 1:
            vals = [np.float32(vals[i] + vals[i + h]) for i in range(h)]
            h //= 2
        want = np.float32(np.sqrt(vals[0]))
        adj = list(sq)
        while len(adj) > 1:
            adj = [np.float32(adj[2 * i] + adj[2 * i + 1]) for i in range(len(adj) // 2)]
        adjacent = np.float32(np.sqrt(adj[0]))
        wide = np.float32(np.sqrt(np.sum(np.asarray(x, np.float64) ** 2)))
        if adjacent != want and wide != want:
            break
    else:
        pytest.fail("no row separates the tree order from its alternatives")
    got = quantize.norm_fp32(x[None])[0]
    assert got.view(np.uint32) == want.view(np.uint32)
    assert got != adjacent and got != wide


def test_decision_rule_ties_go_up():
    t = np.array([-0.5, 0.0, 0.5], np.float32)
    u = np.array([-1.0, -0.5, -0.25, 0.0, 0.25, 0.5, 0.75, 0.5 - 2e-7])
    idx, tie = quantize.indices_for(u, t)
    assert idx.tolist() == [0, 1, 1, 2, 2, 3, 3, 2]
    assert tie.tolist() == [False, True, False, True, False, True, False, True]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_quantize_recovers_planted_indices(D, bits):
    """Rows built as n R^T c[idx] (far from every boundary) must quantize back to idx exactly."""
    rng = np.random.default_rng(D * 10 + bits)
    cb = codebook.codebook(D, bits, "beta")
    R = rotation.rotation_matrix(0, D)
    idx = rng.integers(0, 1 << bits, size=(64, D))
    u = cb.centroids[idx]
    u /= np.linalg.norm(u, axis=1, keepdims=True)    # unit rows whose coordinates sit near centroids
    x = (u @ R) * 40.0                                # x = n R^T u
    x16 = x.astype(np.float16)
    got, n, tie = quantize.quantize_rows(x16, cb.boundaries32, 0)
    # renormalising moves every coordinate by the same factor; compare against the decision on u
    want, _ = quantize.indices_for(u, cb.boundaries32)
    # fp16 rounding of x moves u by ~1e-5; wherever u is 1e-4 clear of every boundary the
    # decision is fixed by u alone
    margin = np.min(np.abs(u[..., None] - cb.boundaries32.astype(np.float64)), axis=-1)
    clear = margin > 1e-4
    assert clear.mean() > (0.5 if bits == 8 else 0.9)
    assert np.array_equal(got[clear], want[clear])
    assert np.allclose(n, 40.0, rtol=1e-3)
    # the wrong rotation direction or the wrong seed does not reproduce them
    wrong, _, _ = quantize.quantize_rows(((u @ R.T) * 40.0).astype(np.float16), cb.boundaries32, 0)
    assert np.mean(wrong == want) < 0.5
    other, _, _ = quantize.quantize_rows(x16, cb.boundaries32, 1)
    assert np.mean(other == want) < 0.5


def test_zero_row():
    cb = codebook.codebook(128, 4, "beta")
    idx, n, tie = quantize.quantize_rows(np.zeros((1, 128), np.float16), cb.boundaries32, 0)
    assert idx.tolist() == [[8] * 128] and n[0] == 0.0
    reg = quantize.pack_region(idx[0], n[0], 4)
    assert reg == bytes([0x88] * 64) + bytes(4)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_dequant_spec_vs_plain(D, bits, rng):
    cb = codebook.codebook(D, bits, "beta")
    idx = rng.integers(0, 1 << bits, size=(50, D))
    n = (rng.random(50) * 30).astype(np.float32)
    spec = quantize.dequantize_spec(idx, n, cb.centroids32, 0).astype(np.float64)
    plain = quantize.dequantize_plain(idx, n, cb.centroids32, 0)
    ulp = np.spacing(np.abs(plain).astype(np.float32)).astype(np.float64)
    # four fp32 roundings (1/sqrt(D), n * that, z, the product) of at most half an ulp each,
    # plus fp64 noise of the dense route where the exact value is 0
    assert np.all(np.abs(spec - plain) <= 4 * ulp + 1e-12 * n[:, None])


@pytest.mark.parametrize("bits, min_cos", [(2, 0.92), (3, 0.975), (4, 0.993), (8, 0.9999)])
def test_reconstruction_quality_tracks_codebook_mse(bits, min_cos):
    """Quantize + dequantize random rows: relative error matches D * MSE; cosine loosely as printed."""
    D = 128
    rng = np.random.default_rng(bits)
    cb = codebook.codebook(D, bits, "beta")
    x16 = rng.standard_normal((3000, D)).astype(np.float16)
    idx, n, _ = quantize.quantize_rows(x16, cb.boundaries32, 0)
    xh = quantize.dequantize_plain(idx, n, cb.centroids32, 0)
    x = x16.astype(np.float64)
    rel = np.mean(np.sum((x - xh) ** 2, 1) / np.sum(x * x, 1))
    assert abs(rel - D * cb.mse) < 0.05 * D * cb.mse
    cos = np.mean(np.sum(x * xh, 1) / (np.linalg.norm(x, axis=1) * np.linalg.norm(xh, axis=1)))
    assert cos > min_cos


def test_append_rows_both_packers_agree_and_address_slots(rng):
    D, H, kb, vb, bs = 64, 3, 3, 2, 16
    ck, cv = codebook.codebook(D, kb), codebook.codebook(D, vb)
    sb = quantize.slot_bytes(D, kb, vb)
    nblk = 4
    k = rng.standard_normal((20, H, D)).astype(np.float16)
    v = rng.standard_normal((20, H, D)).astype(np.float16)
    sm = rng.permutation(nblk * bs)[:20]
    sm[3] = -1
    for stride in (sb, 64):
        if stride < sb:
            continue
        p1 = np.full(nblk * bs * H * stride, 0xAB, np.uint8)
        p2 = p1.copy()
        quantize.append_rows(p1, k, v, sm, ck.boundaries32, cv.boundaries32, kb, vb, 0, stride)
        quantize.append_rows_fast(p2, k, v, sm, ck.boundaries32, cv.boundaries32, kb, vb, 0, stride)
        assert np.array_equal(p1, p2)
        pg = p1.reshape(nblk, bs, H, stride)
        for t in (0, 5, 19):
            s = sm[t]
            (ki, kn), (vi, vn) = quantize.read_slot(p1, s, 2, H, D, kb, vb, stride)
            i_ref, n_ref, _ = quantize.quantize_rows(k[t, 2], ck.boundaries32, 0)
            assert np.array_equal(ki, i_ref) and kn == n_ref
            assert bytes(pg[s // bs, s % bs, 2, :sb]) == bytes(p1[(s * H + 2) * stride:(s * H + 2) * stride + sb])
        assert np.all(pg.reshape(-1, H, stride)[np.setdiff1d(np.arange(nblk * bs), sm)] == 0xAB)


# ============================================================================================
# Attention
# ============================================================================================
def _tiny_cache(rng, D, H_kv, kb, vb, L, bs=16, nblk=None, seed=0):
    ck, cv = codebook.codebook(D, kb), codebook.codebook(D, vb)
    nb = (L + bs - 1) // bs
    nblk = nblk or nb + 3
    bt = rng.permutation(nblk)[:nb]
    k = rng.standard_normal((L, H_kv, D)).astype(np.float16)
    v = rng.standard_normal((L, H_kv, D)).astype(np.float16)
    pos = np.arange(L)
    slots = bt[pos // bs] * bs + pos % bs
    pages = np.zeros(nblk * bs * H_kv * quantize.slot_bytes(D, kb, vb), np.uint8)
    quantize.append_rows_fast(pages, k, v, slots, ck.boundaries32, cv.boundaries32, kb, vb, seed)
    layer = dict(D=D, H_kv=H_kv, block_size=bs, k_bits=kb, v_bits=vb, seed=seed)
    return layer, pages, bt, k, v, ck, cv


@pytest.mark.parametrize("D, H_kv, G, kb, vb, L, ns", [
    (64, 1, 1, 4, 4, 1, 0), (64, 2, 2, 8, 8, 37, 0), (128, 1, 4, 4, 4, 50, 4),
    (128, 2, 3, 3, 2, 17, 2), (128, 1, 8, 8, 4, 64, 4), (64, 1, 1, 2, 2, 5, 5)])
def test_attention_routes_agree(D, H_kv, G, kb, vb, L, ns, rng):
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, kb, vb, L)
    q = rng.standard_normal((1, H_kv * G, D)).astype(np.float16)
    sk = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    sv = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    args = (q, pages, bt[None], np.array([L]), layer, ck.centroids32, cv.centroids32, sk, sv, ns)
    a = attention.decode_attention(*args)
    b = attention.decode_attention_rotated(*args)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_attention_special_cases(rng):
    D, H_kv = 128, 2
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, 4, 4, 40)
    q = rng.standard_normal((1, 4, D)).astype(np.float16)
    run = lambda q_, L, **kw: attention.decode_attention(q_, pages, bt[None], np.array([L]), layer,
                                                         ck.centroids32, cv.centroids32, **kw)
    pos = np.arange(40)
    slots = bt[pos // 16] * 16 + pos % 16
    _, _, v_idx, v_n = quantize.read_slots(pages, slots, H_kv, D, 4, 4)
    vhat = quantize.dequantize_plain(v_idx, v_n, cv.centroids32, 0)      # [40, H_kv, D]
    # L = 1: the output is the single dequantized value row
    o = run(q, 1)
    np.testing.assert_allclose(o[0, 0], vhat[0, 0], atol=1e-12)
    np.testing.assert_allclose(o[0, 3], vhat[0, 1], atol=1e-12)
    # q = 0: uniform weights -> mean of the value rows
    o = run(np.zeros_like(q), 40)
    np.testing.assert_allclose(o[0, 1], vhat[:, 0].mean(0), atol=1e-12)
    np.testing.assert_allclose(o[0, 2], vhat[:, 1].mean(0), atol=1e-12)
    # L = 0: zero output
    assert np.all(run(q, 0) == 0)


def test_attention_all_sinks_is_textbook_softmax_attention(rng):
    import torch
    D, H_kv, G, L = 64, 2, 3, 9
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, 4, 4, L)
    q = rng.standard_normal((1, H_kv * G, D)).astype(np.float16)
    sk = rng.standard_normal((1, L, H_kv, D)).astype(np.float16)
    sv = rng.standard_normal((1, L, H_kv, D)).astype(np.float16)
    o = attention.decode_attention(q, pages, bt[None], np.array([L]), layer, ck.centroids32,
                                   cv.centroids32, sk, sv, n_sink=L)
    # library route: torch scaled_dot_product_attention in fp64 on the CPU, GQA by repetition
    Q = torch.from_numpy(q.astype(np.float64)).reshape(1, H_kv * G, 1, D)
    K = torch.from_numpy(sk[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    V = torch.from_numpy(sv[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).reshape(1, H_kv * G, D).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_attention_identical_keys_and_shift(rng):
    D = 64
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, 1, 4, 4, 20)
    # rewrite every slot's K region with the same row -> weights uniform -> mean of values
    pos = np.arange(20)
    slots = bt[pos // 16] * 16 + pos % 16
    k_same = np.repeat(k[:1], 20, axis=0)
    quantize.append_rows_fast(pages, k_same, v, slots, ck.boundaries32, cv.boundaries32, 4, 4, 0)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    o = attention.decode_attention(q, pages, bt[None], np.array([20]), layer, ck.centroids32, cv.centroids32)
    _, _, v_idx, v_n = quantize.read_slots(pages, slots, 1, D, 4, 4)
    vhat = quantize.dequantize_plain(v_idx, v_n, cv.centroids32, 0)
    np.testing.assert_allclose(o[0, 0], vhat[:, 0].mean(0), atol=1e-12)


# ============================================================================================
# Hot window (turboquant-pro 1.4.2, "Streaming cache" and "Fused CUDA decode"; tq-kv, "3-Fix for
# GGUF Models": the current token kept lossless): the last w positions come from fp16 rows.
# ============================================================================================
def _window_rows(rng, w_cap, H_kv, D, B=1):
    wk = rng.standard_normal((B, w_cap, H_kv, D)).astype(np.float16)
    wv = rng.standard_normal((B, w_cap, H_kv, D)).astype(np.float16)
    return wk, wv


@pytest.mark.parametrize("D, H_kv, G, kb, vb, L, ns, w", [
    (64, 1, 1, 4, 4, 1, 0, 1), (64, 2, 2, 8, 8, 37, 0, 5), (128, 1, 4, 4, 4, 50, 4, 16),
    (128, 2, 3, 3, 2, 17, 2, 15), (64, 1, 1, 2, 2, 5, 5, 0), (128, 1, 8, 8, 4, 64, 0, 63)])
def test_attention_routes_agree_with_window(D, H_kv, G, kb, vb, L, ns, w, rng):
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, kb, vb, L)
    q = rng.standard_normal((1, H_kv * G, D)).astype(np.float16)
    sk = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    sv = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    wk, wv = _window_rows(rng, max(w, 1) + 3, H_kv, D)
    args = (q, pages, bt[None], np.array([L]), layer, ck.centroids32, cv.centroids32, sk, sv, ns)
    kw = dict(win_k16=wk, win_v16=wv, win_lens=np.array([w]))
    a = attention.decode_attention(*args, **kw)
    b = attention.decode_attention_rotated(*args, **kw)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_attention_sinks_and_window_cover_everything_is_textbook(rng):
    import torch
    D, H_kv, G, L, ns = 64, 2, 3, 11, 3
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, 4, 4, L)
    q = rng.standard_normal((1, H_kv * G, D)).astype(np.float16)
    sk = rng.standard_normal((1, ns, H_kv, D)).astype(np.float16)
    sv = rng.standard_normal((1, ns, H_kv, D)).astype(np.float16)
    wk, wv = _window_rows(rng, L - ns + 2, H_kv, D)
    o = attention.decode_attention(q, pages, bt[None], np.array([L]), layer, ck.centroids32,
                                   cv.centroids32, sk, sv, n_sink=ns, win_k16=wk, win_v16=wv,
                                   win_lens=np.array([L - ns]))
    Kall = np.concatenate([sk[0], wk[0, :L - ns]]).astype(np.float64)   # [L, H_kv, D]
    Vall = np.concatenate([sv[0], wv[0, :L - ns]]).astype(np.float64)
    Q = torch.from_numpy(q.astype(np.float64)).reshape(1, H_kv * G, 1, D)
    K = torch.from_numpy(Kall).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    V = torch.from_numpy(Vall).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).reshape(1, H_kv * G, D).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_attention_window_order_and_ignored_slots(rng):
    D, H_kv, G, L, ns, w = 128, 1, 4, 45, 2, 9
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, 4, 4, L)
    q = rng.standard_normal((1, G, D)).astype(np.float16)
    sk = rng.standard_normal((1, ns, H_kv, D)).astype(np.float16)
    sv = rng.standard_normal((1, ns, H_kv, D)).astype(np.float16)
    wk, wv = _window_rows(rng, w, H_kv, D)
    run = lambda pg, wk_, wv_: attention.decode_attention(
        q, pg, bt[None], np.array([L]), layer, ck.centroids32, cv.centroids32, sk, sv, ns,
        win_k16=wk_, win_v16=wv_, win_lens=np.array([w]))
    o = run(pages, wk, wv)
    perm = rng.permutation(w)
    np.testing.assert_allclose(run(pages, wk[:, perm], wv[:, perm]), o, atol=1e-13)
    # overwrite the page slots of the window positions (and the sink positions): no effect
    sb = quantize.slot_bytes(D, 4, 4)
    pg = pages.copy()
    for p in list(range(ns)) + list(range(L - w, L)):
        s = bt[p // 16] * 16 + p % 16
        pg[s * H_kv * sb:(s + 1) * H_kv * sb] = rng.integers(0, 256, H_kv * sb, dtype=np.uint8)
    np.testing.assert_allclose(run(pg, wk, wv), o, atol=0)
    # but a packed position just below the window does matter
    s = bt[(L - w - 1) // 16] * 16 + (L - w - 1) % 16
    pg[s * H_kv * sb:(s + 1) * H_kv * sb] = rng.integers(0, 256, H_kv * sb, dtype=np.uint8)
    assert np.abs(run(pg, wk, wv) - o).max() > 1e-6


def test_attention_zero_query_averages_every_segment(rng):
    D, H_kv, G, L, ns, w = 64, 2, 2, 30, 3, 7
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, 8, 4, L)
    sk = rng.standard_normal((1, ns, H_kv, D)).astype(np.float16)
    sv = rng.standard_normal((1, ns, H_kv, D)).astype(np.float16)
    wk, wv = _window_rows(rng, w + 4, H_kv, D)
    q0 = np.zeros((1, H_kv * G, D), np.float16)
    o = attention.decode_attention(q0, pages, bt[None], np.array([L]), layer, ck.centroids32,
                                   cv.centroids32, sk, sv, ns, win_k16=wk, win_v16=wv,
                                   win_lens=np.array([w]))
    pos = np.arange(ns, L - w)
    slots = bt[pos // 16] * 16 + pos % 16
    _, _, v_idx, v_n = quantize.read_slots(pages, slots, H_kv, D, 8, 4)
    vhat = quantize.dequantize_plain(v_idx, v_n, cv.centroids32, 0)      # [L - ns - w, H_kv, D]
    for h in range(H_kv * G):
        hk = h // G
        rows = np.concatenate([sv[0, :, hk].astype(np.float64), vhat[:, hk],
                               wv[0, :w, hk].astype(np.float64)])
        assert rows.shape[0] == L
        np.testing.assert_allclose(o[0, h], rows.mean(0), atol=1e-12)


# ============================================================================================
# Norm correction (tq-kv, "How It Works": "Lloyd-Max codebook + norm correction", output
# "corrected norm"): the stored norm n / ||c[idx]|| keeps the dequantized row's norm equal to n.
# ============================================================================================
@pytest.mark.parametrize("D, bits", [(64, 2), (128, 4), (128, 3), (64, 8)])
def test_corrected_norm_preserves_the_row_norm(D, bits, rng):
    cb = codebook.codebook(D, bits)
    x = (rng.standard_normal((40, D)) * rng.uniform(0.01, 30, (40, 1))).astype(np.float16)
    x[3] = 0
    idx, n, _ = quantize.quantize_rows(x, cb.boundaries32, 0)
    idx2, nc, _ = quantize.quantize_rows(x, cb.boundaries32, 0, cb.centroids32)
    assert np.array_equal(idx, idx2)
    xhat = quantize.dequantize_plain(idx, nc, cb.centroids32, 0)          # fp64, n' R^T c
    got = np.linalg.norm(xhat, axis=-1)
    exact = np.linalg.norm(x.astype(np.float64), axis=-1)
    # n is within 2.5 ulp of the exact norm, ||c|| within 2.5 ulp, the division 0.5 ulp
    ulp = np.spacing(exact.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - exact) <= 6 * ulp + 1e-300)
    assert nc[3] == 0 and n[3] == 0
    # without the correction the dequantized norm is off by the codebook's norm error
    plain = np.linalg.norm(quantize.dequantize_plain(idx, n, cb.centroids32, 0), axis=-1)
    assert np.max(np.abs(plain[exact > 0] / exact[exact > 0] - 1)) > 1e-4


def test_corrected_norm_by_brute_force(rng):
    # the fp32 tree and operations written out element by element for one row
    D = 16
    c32 = np.sort(rng.standard_normal(4)).astype(np.float32)
    idx = rng.integers(0, 4, D)
    n = np.float32(3.25)
    vals = [np.float32(c32[i]) * np.float32(c32[i]) for i in idx]
    h = D // 2
    while h >= 1:
        vals = [np.float32(vals[i] + vals[i + h]) for i in range(h)]
        h //= 2
    want = np.float32(n / np.float32(np.sqrt(vals[0])))
    got = quantize.corrected_norm(np.array([n]), idx[None], c32)[0]
    assert got.view(np.uint32) == want.view(np.uint32)


# ============================================================================================
# Several queries per sequence (a verified draft or a prompt chunk): the last T positions are the
# queries, each attending the positions up to its own (causal).  Pinned against the textbook
# masked attention over the dequantized rows, not against the single-query oracle it calls.
# ============================================================================================
@pytest.mark.parametrize("D, H_kv, G, kb, vb, L, T, ns", [
    (64, 2, 2, 4, 4, 23, 4, 3), (128, 1, 4, 8, 4, 40, 2, 0), (64, 1, 3, 4, 8, 9, 3, 4)])
def test_multi_query_is_causal_masked_attention(D, H_kv, G, kb, vb, L, T, ns, rng):
    import torch
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, kb, vb, L)
    Hq = H_kv * G
    q = rng.standard_normal((1, T, Hq, D)).astype(np.float16)
    sk = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    sv = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    o = attention.decode_attention_multi(q, pages, bt[None], np.array([L]), layer, ck.centroids32,
                                         cv.centroids32, sk, sv, n_sink=ns)
    pos = np.arange(ns, L)
    slots = bt[pos // 16] * 16 + pos % 16
    k_idx, k_n, v_idx, v_n = quantize.read_slots(pages, slots, H_kv, D, kb, vb)
    Kall = np.concatenate([sk[0, :ns].astype(np.float64), quantize.dequantize_plain(k_idx, k_n, ck.centroids32, 0)])
    Vall = np.concatenate([sv[0, :ns].astype(np.float64), quantize.dequantize_plain(v_idx, v_n, cv.centroids32, 0)])
    Q = torch.from_numpy(q[0].astype(np.float64)).permute(1, 0, 2)[None]            # [1, Hq, T, D]
    K = torch.from_numpy(Kall).permute(1, 0, 2).repeat_interleave(G, 0)[None]       # [1, Hq, L, D]
    V = torch.from_numpy(Vall).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    qpos = torch.arange(L - T, L)[:, None]
    mask = torch.arange(L)[None, :] <= qpos                                          # [T, L]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
    np.testing.assert_allclose(o[0], ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_multi_query_more_queries_than_tokens(rng):
    # queries at negative positions see nothing (zero output); the others are causal as usual
    D, H_kv, G, L, T = 64, 1, 2, 2, 4
    layer, pages, bt, k, v, ck, cv = _tiny_cache(rng, D, H_kv, 4, 4, L)
    q = rng.standard_normal((1, T, H_kv * G, D)).astype(np.float16)
    o = attention.decode_attention_multi(q, pages, bt[None], np.array([L]), layer, ck.centroids32,
                                         cv.centroids32)
    assert np.all(o[0, :2] == 0)
    _, _, v_idx, v_n = quantize.read_slots(pages, bt[:1] * 16 + np.arange(2), H_kv, D, 4, 4)
    vhat = quantize.dequantize_plain(v_idx, v_n, cv.centroids32, 0)
    np.testing.assert_allclose(o[0, 2], np.broadcast_to(vhat[0, 0], (H_kv * G, D)), atol=1e-12)  # one token
    assert np.abs(o[0, 3] - o[0, 2]).max() > 1e-6


# ============================================================================================
# Per-token mean removal (tq-kv, "How It Works": the per-token mean removal stage and the mean in
# the output record): mu is stored after the norm and added back on dequantization.
# ============================================================================================
def test_mean_removal_constant_row_is_exact():
    D, bits = 64, 3
    cb = codebook.codebook(D, bits)
    x = np.full((2, D), [[1.375], [-0.046875]], np.float16)
    idx, n, tie, mu = quantize.quantize_rows(x, cb.boundaries32, 0, mean=True)
    assert np.all(idx == (1 << bits) // 2) and np.all(n == 0)
    assert np.array_equal(mu, x[:, 0].astype(np.float32))
    xhat = quantize.dequantize_spec(idx, n, cb.centroids32, 0, mu)
    assert np.array_equal(xhat, x.astype(np.float32))


def test_mean_removal_shift_moves_only_the_mean(rng):
    # integer-valued rows: every sum is exact, so a shift by 8 changes mu by exactly 8 and
    # leaves the centred row, its norm and its indices unchanged
    D = 128
    cb = codebook.codebook(D, 4)
    x = rng.integers(-20, 21, (16, D)).astype(np.float16)
    a = quantize.quantize_rows(x, cb.boundaries32, 0, mean=True)
    b = quantize.quantize_rows((x + 8).astype(np.float16), cb.boundaries32, 0, mean=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(b[3], a[3] + np.float32(8))


def test_mean_removal_by_brute_force(rng):
    # the fp32 operations written out element by element for one row
    D = 16
    x = (rng.standard_normal(D) * 3).astype(np.float16)
    vals = [np.float32(v) for v in x]
    h = D // 2
    while h >= 1:
        vals = [np.float32(vals[i] + vals[i + h]) for i in range(h)]
        h //= 2
    mu = np.float32(vals[0] / np.float32(D))
    d = [np.float32(np.float32(v) - mu) for v in x]
    sq = [np.float32(e * e) for e in d]
    h = D // 2
    while h >= 1:
        sq = [np.float32(sq[i] + sq[i + h]) for i in range(h)]
        h //= 2
    n = np.float32(np.sqrt(sq[0]))
    assert quantize.row_mean(x[None])[0].view(np.uint32) == mu.view(np.uint32)
    assert quantize.centered_norm(x[None], np.array([mu]))[0].view(np.uint32) == n.view(np.uint32)


def test_mean_removal_reconstructs_offset_rows_better(rng):
    D, bits = 128, 2
    cb = codebook.codebook(D, bits)
    x = (rng.standard_normal((64, D)) * 0.3 + 2.0).astype(np.float16)   # a large common offset
    xf = x.astype(np.float64)
    cos = lambda a: np.sum(a * xf, -1) / (np.linalg.norm(a, axis=-1) * np.linalg.norm(xf, axis=-1))
    idx, n, _ = quantize.quantize_rows(x, cb.boundaries32, 0)
    plain = quantize.dequantize_plain(idx, n, cb.centroids32, 0)
    idx_m, n_m, _, mu = quantize.quantize_rows(x, cb.boundaries32, 0, mean=True)
    centred = quantize.dequantize_plain(idx_m, n_m, cb.centroids32, 0, mu)
    err = lambda a: np.linalg.norm(a - xf, axis=-1) / np.linalg.norm(xf, axis=-1)
    assert np.median(err(centred)) < 0.5 * np.median(err(plain))
    assert np.all(cos(centred) > 0.99)
    # the spec route agrees with the plain one within a few ulp
    spec = quantize.dequantize_spec(idx_m, n_m, cb.centroids32, 0, mu)
    np.testing.assert_allclose(spec, centred, rtol=0, atol=4 * np.spacing(np.float32(np.abs(centred).max())))


@pytest.mark.parametrize("D, H_kv, G, kb, vb, L, ns", [(64, 2, 2, 4, 8, 37, 0), (128, 1, 4, 2, 3, 50, 4)])
def test_attention_routes_agree_with_mean_removal(D, H_kv, G, kb, vb, L, ns, rng):
    ck, cv = codebook.codebook(D, kb), codebook.codebook(D, vb)
    nb = (L + 15) // 16
    bt = rng.permutation(nb + 2)[:nb]
    k = (rng.standard_normal((L, H_kv, D)) + rng.standard_normal((L, H_kv, 1)) * 3).astype(np.float16)
    v = (rng.standard_normal((L, H_kv, D)) + rng.standard_normal((L, H_kv, 1)) * 3).astype(np.float16)
    slots = bt[np.arange(L) // 16] * 16 + np.arange(L) % 16
    pages = np.zeros((nb + 2) * 16 * H_kv * quantize.slot_bytes(D, kb, vb, True), np.uint8)
    quantize.append_rows_fast(pages, k, v, slots, ck.boundaries32, cv.boundaries32, kb, vb, 0, mean=True)
    layer = dict(D=D, H_kv=H_kv, block_size=16, k_bits=kb, v_bits=vb, seed=0, mean=True)
    q = rng.standard_normal((1, H_kv * G, D)).astype(np.float16)
    sk = rng.standard_normal((1, max(ns, 1), H_kv, D)).astype(np.float16)
    args = (q, pages, bt[None], np.array([L]), layer, ck.centroids32, cv.centroids32, sk, sk, ns)
    np.testing.assert_allclose(attention.decode_attention(*args), attention.decode_attention_rotated(*args),
                               atol=1e-12, rtol=0)
