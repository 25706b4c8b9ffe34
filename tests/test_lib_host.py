"""CPU-only checks of the HIP library: it loads, exports every declared symbol, and its host-side
set-up (slot bytes, rotation signs, Lloyd-Max codebooks, argument validation) matches the oracle.
No kernel is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import codebook as ocb
from oracle import quantize as oq
from oracle import rotation as orot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import packed_decode_attention_amd._lib as L
    return L


def test_library_exports_every_declared_symbol(lib):
    with open(os.path.join(ROOT, "include", "tq.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", header))
    assert declared == set(lib.EXPORTS)
    so = ctypes.CDLL(lib.LIB_PATH)
    for name in declared:
        assert hasattr(so, name), name
    with open(os.path.join(ROOT, "include", "tq_probe.h")) as f:
        probe = set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", f.read()))
    assert probe == set(lib.PROBE_EXPORTS)
    for name in probe:
        assert hasattr(so, name), name


def test_slot_bytes(lib):
    for D in (64, 128, 256, 1024):
        for kb in range(1, 9):
            for vb in range(1, 9):
                assert lib.tq_slot_bytes(D, kb, vb) == oq.slot_bytes(D, kb, vb)
                for flags in range(8):  # norm correction, mean removal, QJL key sketch
                    assert lib.tq_slot_bytes_ex(D, kb, vb, flags) == oq.slot_bytes(D, kb, vb, bool(flags & 2),
                                                                                 bool(flags & 4))
    with pytest.raises(lib.TqError):
        lib.tq_slot_bytes(128, 9, 4)
    with pytest.raises(lib.TqError):
        lib.tq_slot_bytes_ex(128, 4, 4, 8)
    with pytest.raises(lib.TqError):
        lib.tq_slot_bytes_ex(100, 4, 4, 4)   # the sketch needs D a multiple of 8


def test_rht_signs_match_oracle(lib):
    for D in (64, 128, 1000):
        for seed in (0, 1, 12345, 2 ** 63 + 7):
            assert lib.tq_rht_signs(D, seed).tolist() == orot.signs(seed, D).astype(int).tolist()


@pytest.mark.parametrize("family", ["beta", "gaussian"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_build_codebook_matches_oracle(lib, family, D, bits):
    c, t, c64, t64, mse = lib.tq_build_codebook(D, bits, family)
    ref = ocb.codebook(D, bits, family)
    np.testing.assert_allclose(c64, ref.centroids, atol=1e-10, rtol=0)
    np.testing.assert_allclose(t64, ref.boundaries, atol=1e-10, rtol=0)
    assert abs(mse - ref.mse) < 1e-12
    # The fp32 arrays the kernels use equal the oracle's, except where the fp64 fixed point lies
    # so close to an fp32 rounding midpoint that the two independent fp64 solves (which agree to
    # about 1e-11 at 256 levels) round to neighbouring floats.  Those rounding ties are 1 ulp apart.
    for got, want64 in ((c, ref.centroids), (t, ref.boundaries)):
        want = want64.astype(np.float32)
        diff = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
        for i in diff:
            a, b = sorted((float(got[i]), float(want[i])))
            assert np.nextafter(np.float32(a), np.float32(np.inf)) == np.float32(b)
            assert abs(want64[i] - 0.5 * (a + b)) < 5e-11
        assert len(diff) <= 4


def test_build_codebook_rejects_bad_arguments(lib):
    with pytest.raises(lib.TqError):
        lib.tq_build_codebook(128, 9, "beta")
    so = lib._lib()
    buf = np.zeros(16, np.float32)
    assert so.tq_build_codebook(128, 4, 7, buf.ctypes.data, buf.ctypes.data, None, None, None) == lib.TQ_ERR_INVALID_ARG
    assert so.tq_build_codebook(128, 4, 0, None, buf.ctypes.data, None, None, None) == lib.TQ_ERR_INVALID_ARG


def _desc(lib, **kw):
    fake = 0x10000  # never dereferenced: validation fails before anything is enqueued
    d = dict(head_dim=128, num_q_heads=32, num_kv_heads=8, block_size=16, k_bits=4, v_bits=4,
             slot_stride=0, flags=0, rht_seed=0, k_centroids=fake, k_boundaries=fake,
             v_centroids=fake, v_boundaries=fake)
    d.update(kw)
    return lib.tq_layer_desc(**d)


def test_argument_validation_before_launch(lib):
    so = lib._lib()
    P = ctypes.c_void_p(0x20000)
    E = lib
    q = lambda d, n=4, **kw: so.tq_quantize_append(ctypes.byref(d), kw.get("k", P), kw.get("v", P),
                                                    kw.get("sm", P), n, kw.get("pages", P), 10, None)
    assert q(_desc(lib, head_dim=96)) == E.TQ_ERR_UNSUPPORTED
    assert q(_desc(lib, k_bits=5)) == E.TQ_ERR_UNSUPPORTED
    assert q(_desc(lib, v_bits=1)) == E.TQ_ERR_UNSUPPORTED
    assert q(_desc(lib, slot_stride=100)) == E.TQ_ERR_INVALID_ARG      # < 136
    assert q(_desc(lib, slot_stride=138)) == E.TQ_ERR_INVALID_ARG      # not a multiple of 4
    assert q(_desc(lib, flags=8)) == E.TQ_ERR_INVALID_ARG              # unknown format flag
    assert q(_desc(lib, flags=4, k_bits=8)) == E.TQ_ERR_UNSUPPORTED    # the sketch is for 2-4-bit keys
    assert q(_desc(lib, flags=4, slot_stride=136)) == E.TQ_ERR_INVALID_ARG  # < 156 with the sketch
    assert q(_desc(lib, flags=2, slot_stride=136)) == E.TQ_ERR_INVALID_ARG  # < 144 with the mean
    assert q(_desc(lib, flags=-1)) == E.TQ_ERR_INVALID_ARG
    assert q(_desc(lib, num_kv_heads=0)) == E.TQ_ERR_INVALID_ARG
    assert q(_desc(lib, block_size=0)) == E.TQ_ERR_INVALID_ARG
    assert q(_desc(lib, k_centroids=0)) == E.TQ_ERR_INVALID_ARG
    assert q(_desc(lib), k=None) == E.TQ_ERR_INVALID_ARG
    assert q(_desc(lib), n=-1) == E.TQ_ERR_INVALID_ARG
    assert q(_desc(lib), n=0, k=None) == E.TQ_OK                       # nothing to do
    assert so.tq_quantize_append(None, P, P, P, 1, P, 1, None) == E.TQ_ERR_INVALID_ARG

    def dec(d, ws_bytes=1 << 40, n_sink=0, sk=None, B=4, max_len=100, bt=P, mb=7):
        return so.tq_paged_decode_attention(ctypes.byref(d), P, P, 100, bt, mb, P, B, max_len, sk, sk,
                                            n_sink, 0.0, P, P, ws_bytes, None)
    assert dec(_desc(lib, num_q_heads=30)) == E.TQ_ERR_INVALID_ARG      # 30 % 8 != 0
    assert dec(_desc(lib, num_q_heads=72)) == E.TQ_ERR_UNSUPPORTED      # G = 9 > 8
    assert dec(_desc(lib), ws_bytes=16) == E.TQ_ERR_WORKSPACE
    assert dec(_desc(lib), n_sink=4) == E.TQ_ERR_INVALID_ARG            # sinks without arrays
    assert dec(_desc(lib), n_sink=129, sk=P) == E.TQ_ERR_UNSUPPORTED
    assert dec(_desc(lib), mb=6) == E.TQ_ERR_INVALID_ARG                # 6 * 16 < 100 tokens
    assert dec(_desc(lib), bt=None) == E.TQ_ERR_INVALID_ARG
    assert dec(_desc(lib), B=0) == E.TQ_OK
    assert dec(_desc(lib), B=-1) == E.TQ_ERR_INVALID_ARG
    # a split grid beyond 32-bit workgroup counts
    assert dec(_desc(lib), B=65535, max_len=2 ** 31 - 1, mb=2 ** 27) == E.TQ_ERR_UNSUPPORTED

    def deca(d, B=4, kn=P, ws_bytes=1 << 40, mb=7, pages=P):
        return so.tq_paged_decode_attention_append(ctypes.byref(d), P, kn, kn, pages, 100, P, mb, P, B,
                                                   100, 0.0, P, P, ws_bytes, None)
    # formats served by neither the block kernel nor the split kernel's staged instances
    assert deca(_desc(lib, v_bits=3)) == E.TQ_ERR_UNSUPPORTED             # 3-bit values: vector kernel
    assert deca(_desc(lib, head_dim=64, k_bits=2)) == E.TQ_ERR_UNSUPPORTED  # D = 64, 2-bit keys
    assert deca(_desc(lib, k_bits=8, block_size=8)) == E.TQ_ERR_UNSUPPORTED  # runs of 16 split by blocks
    assert deca(_desc(lib, flags=1)) == E.TQ_ERR_UNSUPPORTED              # norm correction
    assert deca(_desc(lib, k_bits=8, flags=2)) == E.TQ_ERR_UNSUPPORTED    # mean removal
    assert deca(_desc(lib, flags=4, slot_stride=160)) == E.TQ_ERR_UNSUPPORTED  # QJL keys
    assert deca(_desc(lib, num_q_heads=72)) == E.TQ_ERR_UNSUPPORTED
    assert deca(_desc(lib), B=513) == E.TQ_ERR_UNSUPPORTED                # above TQ_APPEND_MAX_SEQS
    assert deca(_desc(lib), kn=None) == E.TQ_ERR_INVALID_ARG
    assert deca(_desc(lib), pages=None) == E.TQ_ERR_INVALID_ARG
    assert deca(_desc(lib), ws_bytes=16) == E.TQ_ERR_WORKSPACE
    assert deca(_desc(lib), mb=6) == E.TQ_ERR_INVALID_ARG                 # 6 * 16 < 100 tokens
    assert deca(_desc(lib), B=0, kn=None) == E.TQ_OK                      # nothing to do
    assert deca(_desc(lib), B=-1) == E.TQ_ERR_INVALID_ARG

    def decw(d, cap=16, wk=P, wl=P, B=4):
        return so.tq_paged_decode_attention_window(ctypes.byref(d), P, P, 100, P, 7, P, B, 100, None,
                                                   None, 0, wk, wk, wl, cap, 0.0, P, P, 1 << 40, None)
    assert decw(_desc(lib), cap=1025) == E.TQ_ERR_UNSUPPORTED            # capacity above 1024
    assert decw(_desc(lib), cap=-1) == E.TQ_ERR_INVALID_ARG
    assert decw(_desc(lib), wk=None) == E.TQ_ERR_INVALID_ARG             # window without arrays
    assert decw(_desc(lib), wl=None) == E.TQ_ERR_INVALID_ARG
    assert decw(_desc(lib), cap=0, wk=None, wl=None, B=0) == E.TQ_OK     # no window, nothing to do
    assert decw(_desc(lib, num_q_heads=72)) == E.TQ_ERR_UNSUPPORTED

    def decm(d, T=2, ws_bytes=1 << 40, B=4, n_sink=0, sk=None):
        return so.tq_paged_decode_attention_multi(ctypes.byref(d), P, T, P, 100, P, 7, P, B, 100, sk,
                                                  sk, n_sink, 0.0, P, P, ws_bytes, None)
    assert decm(_desc(lib), T=0) == E.TQ_ERR_INVALID_ARG
    assert decm(_desc(lib), T=65) == E.TQ_ERR_UNSUPPORTED                 # above TQ_MAX_QUERIES
    assert decm(_desc(lib), ws_bytes=16) == E.TQ_ERR_WORKSPACE
    assert decm(_desc(lib), n_sink=2) == E.TQ_ERR_INVALID_ARG             # sinks without arrays
    assert decm(_desc(lib, num_q_heads=72)) == E.TQ_ERR_UNSUPPORTED
    assert decm(_desc(lib), B=0) == E.TQ_OK
    assert so.tq_paged_decode_attention_multi(ctypes.byref(_desc(lib)), P, 2, P, 100, P, 2 ** 27, P, 65535,
                                              2 ** 31 - 1, None, None, 0, 0.0, P, P, 1 << 40,
                                              None) == E.TQ_ERR_UNSUPPORTED

    dq = lambda d, n=3: so.tq_dequantize_rows(ctypes.byref(d), P, 10, P, n, P, P, None)
    assert dq(_desc(lib, head_dim=256)) == E.TQ_ERR_UNSUPPORTED
    assert dq(_desc(lib), n=-2) == E.TQ_ERR_INVALID_ARG
    assert dq(_desc(lib), n=0) == E.TQ_OK
    assert dq(_desc(lib), n=2 ** 35) == E.TQ_ERR_UNSUPPORTED                # grid beyond 2^31 workgroups
    assert so.tq_dequantize_rows(ctypes.byref(_desc(lib)), None, 10, P, 3, P, P, None) == E.TQ_ERR_INVALID_ARG


def test_workspace_bytes(lib):
    d = _desc(lib)
    so = lib._lib()
    a = so.tq_decode_workspace_bytes(ctypes.byref(d), 16, 32769)
    b = so.tq_decode_workspace_bytes(ctypes.byref(d), 16, 100)
    assert a >= b > 0
    # block kernel: partials (m, l, acc[D]) per sequence, kv head, piece (2 * 256 / 16 + 2 = 34
    # for 16 sequences) and query head, rounded up to 256 bytes, then a piece count per sequence
    assert a >= 16 * 8 * 34 * 4 * 130 * 4 + 16 * 4 and (a - 16 * 4) % 256 == 0
    # the split kernel (another format): partials only, per sequence, query head and split
    c = so.tq_decode_workspace_bytes(ctypes.byref(_desc(lib, k_bits=8)), 16, 32769)
    assert c >= 16 * 8 * 4 * 130 * 4 and c % (32 * 130 * 4) == 0
    assert so.tq_decode_workspace_bytes(ctypes.byref(_desc(lib, head_dim=80)), 16, 100) == 0


def test_multi_query_workspace_bytes(lib):
    so = lib._lib()
    d = _desc(lib)                                       # G = 4: two queries per launch
    one = so.tq_decode_workspace_bytes(ctypes.byref(d), 16, 32769)
    assert so.tq_decode_multi_workspace_bytes(ctypes.byref(d), 16, 32769, 1) == one
    # a launch of two queries is a launch of eight query heads per kv head (its own kernel and
    # split geometry); the launches reuse one workspace, sized for the largest of them
    two = so.tq_decode_workspace_bytes(ctypes.byref(_desc(lib, num_q_heads=64)), 16, 32769)
    assert so.tq_decode_multi_workspace_bytes(ctypes.byref(d), 16, 32769, 2) == two
    assert so.tq_decode_multi_workspace_bytes(ctypes.byref(d), 16, 32769, 8) == two
    assert so.tq_decode_multi_workspace_bytes(ctypes.byref(d), 16, 32769, 7) == max(one, two)  # 2+2+2+1
    g8 = _desc(lib, num_q_heads=64)                      # G = 8: one query per launch
    assert (so.tq_decode_multi_workspace_bytes(ctypes.byref(g8), 4, 1000, 5) ==
            so.tq_decode_workspace_bytes(ctypes.byref(g8), 4, 1000))
    assert so.tq_decode_multi_workspace_bytes(ctypes.byref(d), 16, 100, 0) == 0
    assert so.tq_decode_multi_workspace_bytes(ctypes.byref(d), 16, 100, 65) == 0


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(lib.tq_status_str(s), str) and lib.tq_status_str(s)


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: with the HIP library absent, the first call raises instead of computing."""
    import subprocess
    import sys
    code = ("import packed_decode_attention_amd as tq\n"
            "try:\n"
            "    tq.tq_slot_bytes(128, 4, 4)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('computed')\n")
    env = dict(os.environ, TQ_LIB=str(tmp_path / "absent" / "libtq.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "not built" in r.stdout
