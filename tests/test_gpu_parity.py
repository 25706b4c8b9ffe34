"""GPU parity of the HIP path against the CPU oracle, through the C ABI, on seeded inputs shaped
like the five workloads (reduced sizes the oracle finishes in seconds, several splits and a ragged
tail each) and on the edge cases.  Three levels: packed bytes bit-exact apart from oracle-listed
ties; dequantized rows bit-exact; attention within 1e-3 max-abs and 1e-4 relative L2."""

import numpy as np
import pytest

from packed_decode_attention_amd import workloads as wl

from _parity import Case, check_attention, compare_pages

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS

CASES = {
    "tiny": dict(w=W["tiny"]),
    "qwen-small": dict(w=wl.scaled(W["qwen2.5-0.5b"], num_seqs=3), lens=[1000, 517, 64]),
    "llama-small": dict(w=wl.scaled(W["llama3-8b"], num_seqs=2), lens=[1500, 777]),
    "mistral-small": dict(w=wl.scaled(W["mistral-7b"], num_seqs=3), lens=[900, 3, 130]),
    "mistral-protected": dict(w=wl.scaled(W["mistral-7b"], num_seqs=2), layer=31, lens=[640, 70]),
    "ragged-small": dict(w=wl.scaled(W["ragged"], num_seqs=6), lens=[1, 613, 64, 65, 300, 129]),
    # a power-of-two slot stride (136 -> 256 bytes, the TQ4 page tensor's optional padding) on the
    # staged matrix-core path
    "llama-pow2": dict(w=wl.scaled(W["llama3-8b"], num_seqs=2), lens=[1100, 333], slot_stride=256),
    "edges": dict(w=wl.Workload("edges", 1, 6, 6, 2, 128, 2, 3, 0, block_size=7, n_sink=4,
                                values="normal", tables="fragmented", seed=11),
                  lens=[0, 1, 4, 5, 17, 200], slot_stride=160),
    "gaussian-g5": dict(w=wl.Workload("g5", 1, 3, 10, 2, 64, 4, 8, 0, block_size=32,
                                      values="student_t", seed=12),
                        lens=[333, 96, 1], family="gaussian"),
    # norm-correction format (stored norm n / ||c[idx]||), at each register shape and bit width
    "llama-nc": dict(w=wl.scaled(W["llama3-8b"], num_seqs=2), lens=[1100, 333], norm_correction=True),
    "edges-nc": dict(w=wl.Workload("edges-nc", 1, 6, 6, 2, 128, 2, 3, 0, block_size=7, n_sink=4,
                                   values="normal", tables="fragmented", seed=13),
                     lens=[0, 1, 3, 5, 66, 200], slot_stride=160, norm_correction=True),
    "g5-nc": dict(w=wl.Workload("g5-nc", 1, 3, 10, 2, 64, 8, 4, 0, block_size=32,
                                values="student_t", seed=14),
                  lens=[333, 96, 1], family="gaussian", norm_correction=True),
    # mean-removal format (the row mean after the norm): matrix-core kernel's per-lane path (G = 4,
    # G = 8), the vector kernel (2/3-bit codes, block size 7, padded stride), with norm correction
    "llama-mean": dict(w=wl.scaled(W["llama3-8b"], num_seqs=2), lens=[1100, 333], mean_removal=True),
    "ragged-mean": dict(w=wl.scaled(W["ragged"], num_seqs=3), lens=[700, 65, 1], mean_removal=True),
    "edges-mean": dict(w=wl.Workload("edges-mean", 1, 6, 6, 2, 128, 2, 3, 0, block_size=7, n_sink=4,
                                     values="normal", tables="fragmented", seed=15),
                       lens=[0, 1, 3, 5, 66, 200], slot_stride=160, mean_removal=True),
    "g5-mean-nc": dict(w=wl.Workload("g5-mean-nc", 1, 3, 10, 2, 64, 4, 8, 0, block_size=32,
                                     values="student_t", seed=16),
                       lens=[333, 96, 1], family="gaussian", norm_correction=True, mean_removal=True),
    # QJL key format (1-bit residual sketch of 2-4-bit keys): the matrix-core kernel's residual
    # products at 4 and 8 heads (D = 128) and 5 heads (D = 64) and with block size 7, sinks and a
    # padded stride; the vector kernel (3-bit values); combined with the other two format flags
    "llama-qjl": dict(w=wl.scaled(W["llama3-8b"], num_seqs=2), lens=[1100, 333], qjl=True),
    "llama-qjl-mean": dict(w=wl.scaled(W["llama3-8b"], num_seqs=2), lens=[517, 64], qjl=True,
                           mean_removal=True),
    "ragged-qjl": dict(w=wl.scaled(W["ragged"], num_seqs=3), lens=[700, 65, 1], qjl=True),
    "edges-qjl-mean": dict(w=wl.Workload("edges-qjl", 1, 6, 6, 2, 128, 2, 3, 0, block_size=7, n_sink=4,
                                         values="normal", tables="fragmented", seed=17),
                           lens=[0, 1, 3, 5, 66, 200], slot_stride=160, mean_removal=True, qjl=True),
    "edges-qjl": dict(w=wl.Workload("edges-qjl2", 1, 6, 6, 2, 128, 2, 2, 0, block_size=7, n_sink=4,
                                    values="normal", tables="fragmented", seed=19),
                      lens=[0, 1, 3, 5, 66, 200], slot_stride=160, qjl=True),
    # the whole-block streaming kernel (K4/V4, D = 128, eight kv heads): lengths around run and
    # stage edges, G = 2 with 32-position blocks, G = 3 with more units than workgroups (each
    # workgroup takes several), G = 1 with sinks ending mid-run
    "blk-edges": dict(w=wl.Workload("blk-edges", 1, 10, 32, 8, 128, 4, 4, 0, values="outliers", seed=51),
                      lens=[1, 15, 16, 17, 31, 32, 33, 48, 500, 2047]),
    "blk-g2-bs32": dict(w=wl.Workload("blk-g2", 1, 3, 16, 8, 128, 4, 4, 0, block_size=32, seed=52),
                        lens=[1000, 333, 77]),
    "blk-g3-many": dict(w=wl.Workload("blk-g3", 1, 300, 24, 8, 128, 4, 4, 0, seed=53),
                        lens=list(np.random.default_rng(53).integers(1, 121, 300))),
    "blk-g1-sinks": dict(w=wl.Workload("blk-g1", 1, 4, 8, 8, 128, 4, 4, 0, n_sink=20, seed=54),
                         lens=[700, 33, 21, 5]),
    # the whole-block kernel's K3/V2 instances (the ragged batch's format): G = 8 around run
    # edges with a sequence spread over many workgroups, G = 4 with sinks ending mid-run and
    # fragmented tables, many short sequences (several pieces per workgroup), and one long
    # sequence cut into hundreds of pieces
    "blk32-edges": dict(w=wl.Workload("blk32-edges", 1, 9, 64, 8, 128, 3, 2, 0, values="outliers", seed=61),
                        lens=[1, 15, 16, 17, 33, 48, 500, 2047, 6000]),
    "blk32-g4-sinks": dict(w=wl.Workload("blk32-g4", 1, 4, 32, 8, 128, 3, 2, 0, n_sink=20,
                                         tables="fragmented", seed=62), lens=[700, 33, 21, 5]),
    "blk32-many": dict(w=wl.Workload("blk32-many", 1, 400, 64, 8, 128, 3, 2, 0, seed=63),
                       lens=list(np.random.default_rng(63).integers(1, 200, 400))),
    "blk32-long": dict(w=wl.Workload("blk32-long", 1, 1, 64, 8, 128, 3, 2, 0, values="student_t", seed=64),
                       lens=[20000]),
    # balanced ranges whose pieces exceed one unit of 1024 runs (a 2400-run sequence among 255
    # one-run ones may span at most three workgroups: 1201 runs per workgroup), and workgroups
    # with over a hundred pieces
    "blk32-units": dict(w=wl.Workload("blk32-units", 1, 256, 64, 8, 128, 3, 2, 0, seed=65),
                        lens=[16] * 100 + [38400] + [16] * 155),
    "blk-units": dict(w=wl.Workload("blk-units", 1, 256, 32, 8, 128, 4, 4, 0, seed=66),
                      lens=[16] * 40 + [12999] + [16] * 215),
    # the largest sink count (128): sequences shorter than, equal to and longer than it
    "sinks-max": dict(w=wl.Workload("sinks-max", 1, 4, 8, 2, 128, 4, 4, 0, n_sink=128, values="normal",
                                    seed=20), lens=[100, 128, 129, 700]),
    "g8-v3-qjl": dict(w=wl.Workload("g8-v3-qjl", 1, 3, 16, 2, 128, 4, 3, 0, values="normal", seed=21),
                      lens=[777, 64, 2], qjl=True),  # the vector kernel's 8-head instance
    "g5-qjl-nc": dict(w=wl.Workload("g5-qjl-nc", 1, 3, 10, 2, 64, 4, 8, 0, block_size=32,
                                    values="student_t", seed=18),
                      lens=[333, 96, 1], family="gaussian", norm_correction=True, qjl=True),
}


def _case(name):
    spec = dict(CASES[name])
    return Case(spec.pop("w"), **spec)


@pytest.fixture(scope="module")
def cases():
    return {}


def get(cases, name):
    if name not in cases:
        print(f"[parity] building case {name}", flush=True)
        cases[name] = _case(name)
    return cases[name]


@pytest.mark.parametrize("name", list(CASES))
def test_quantize_bytes(cases, name):
    c = get(cases, name)
    fmt = c.fmt()
    print(f"[parity] quantize {name}: rows={len(c.slots)} H={c.H} D={c.D} K{c.kb}/V{c.vb}", flush=True)
    pages = c.gpu_quantize(fmt).cpu().numpy().reshape(-1)
    ties = compare_pages(pages, c.pages_ref, c.slots, c.H, c.D, c.kb, c.vb, c.slot_stride, c.k_tie, c.v_tie,
                         c.nc_args(), c.mean, c.q_tie)
    assert ties <= max(4, 1e-4 * c.slots.size * c.H * c.D)
    # untouched slots keep their contents
    used = np.zeros(c.num_blocks * c.w.block_size, bool)
    used[c.slots] = True
    assert np.all(pages.reshape(-1, c.H, c.slot_stride)[~used] == 0x5A)


@pytest.mark.parametrize("name", list(CASES))
def test_dequantize_rows_bit_exact(cases, name):
    import torch
    import packed_decode_attention_amd as tq
    c = get(cases, name)
    fmt = c.fmt()
    rng = np.random.default_rng(3)
    slots = rng.choice(c.slots, size=min(257, c.slots.size), replace=False).astype(np.int64)
    print(f"[parity] dequantize {name}: {slots.size} slots", flush=True)
    ko = torch.empty((slots.size, c.H, c.D), dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    tq.tq_dequantize_rows(fmt.desc, c.ref_pages_on_gpu(), c.num_blocks, torch.from_numpy(slots).cuda(), ko, vo)
    torch.cuda.synchronize()
    kr, vr = c.oracle_dequant(slots)
    assert np.array_equal(ko.cpu().numpy().view(np.uint32), kr.view(np.uint32))
    assert np.array_equal(vo.cpu().numpy().view(np.uint32), vr.view(np.uint32))


@pytest.mark.parametrize("name", list(CASES))
def test_decode_attention(cases, name):
    c = get(cases, name)
    fmt = c.fmt()
    print(f"[parity] decode {name}: lens={c.lens.tolist()} Hq={c.Hq} H={c.H} sinks={c.w.n_sink}", flush=True)
    want = c.oracle_decode()
    got, ws = c.gpu_decode(fmt, c.ref_pages_on_gpu())
    check_attention(got, want)
    # same workspace again: results are bit-identical (the decode is deterministic)
    again, _ = c.gpu_decode(fmt, c.ref_pages_on_gpu(), workspace=ws)
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    # On the GPU's own pages: a tie may pick the neighbouring code, which moves that key or value
    # by a whole cell, so only sequences whose packed bytes equal the oracle's are held to the
    # tolerance here (the tie differences themselves are checked by test_quantize_bytes).
    own_pages = c.gpu_quantize(fmt)
    own, _ = c.gpu_decode(fmt, own_pages)
    g = own_pages.cpu().numpy().reshape(-1, c.H, c.slot_stride)[c.slots]
    r = c.pages_ref.reshape(-1, c.H, c.slot_stride)[c.slots]
    same_tok = np.all(g.reshape(len(c.slots), -1) == r.reshape(len(c.slots), -1), axis=1)
    offs = np.concatenate([[0], np.cumsum(c.lens)])
    clean = [b for b in range(len(c.lens)) if np.all(same_tok[offs[b]:offs[b + 1]])]
    print(f"[parity] {name}: sequences without tie differences {clean}", flush=True)
    if clean:
        check_attention(own, want, seqs=clean)
    zero = np.nonzero(c.lens == 0)[0]
    assert np.all(got[zero] == 0)


# Several causal queries per sequence: (case, T).  T * G <= 8 runs as one launch on the kernels'
# 8-head instances; more queries take several launches over the same workspace.  The cases cover
# the matrix-core kernel (G = 4 at T = 1, 2, 3, 5; G = 8; D = 64 with G = 5), the vector kernel
# (edges: G = 3, 2/3-bit codes, block size 7), sinks, and sequences shorter than T.
MULTI = [("llama-small", 1), ("llama-small", 2), ("llama-small", 3), ("llama-small", 5),
         ("mistral-small", 2), ("ragged-small", 3), ("edges", 2), ("gaussian-g5", 2), ("tiny", 4),
         ("llama-mean", 2), ("edges-mean", 3), ("llama-qjl", 2), ("ragged-qjl", 2), ("edges-qjl", 3),
         ("tiny", 64), ("sinks-max", 64),  # 64: the largest query count
         ("blk-g2-bs32", 2), ("blk-g1-sinks", 4),  # two or four queries on the whole-block kernel
         ("blk32-g4-sinks", 2), ("blk32-edges", 2)]  # K3/V2: one launch of eight heads, two of eight


@pytest.mark.parametrize("name,T", MULTI, ids=[f"{n}-T{t}" for n, t in MULTI])
def test_decode_attention_multi_query(cases, name, T):
    c = get(cases, name)
    fmt = c.fmt()
    qm = c.queries_multi(T)
    print(f"[parity] multi-query {name} T={T}: lens={c.lens.tolist()} Hq={c.Hq} H={c.H}", flush=True)
    want = c.oracle_decode_multi(qm)
    got = c.gpu_decode_multi(fmt, c.ref_pages_on_gpu(), qm)
    check_attention(got.reshape(-1, c.Hq, c.D), want.reshape(-1, c.Hq, c.D))
    vis = c.lens[:, None] - T + np.arange(T)[None, :] + 1   # positions each query sees
    assert np.all(got[vis <= 0] == 0)
    if T == 1:  # one query is the single-query call, bit for bit
        assert np.array_equal(qm[:, 0].numpy(), c.q.numpy())
        single, _ = c.gpu_decode(fmt, c.ref_pages_on_gpu())
        assert np.array_equal(got[:, 0].view(np.uint32), single.view(np.uint32))


# Hot-window lengths per sequence (each <= L - min(n_sink, L)) and the window capacity: a window
# per case shape, including windows that hold every non-sink token (no packed tokens left), a
# one-token window (the current token only) and the largest capacity.
WINDOWS = {
    "tiny": ([1], 8),
    "qwen-small": ([200, 517, 0], 600),
    "llama-small": ([64, 0], 100),
    "mistral-small": ([512, 0, 126], 1024),
    "ragged-small": ([1, 100, 0, 65, 17, 128], 130),
    "edges": ([0, 0, 0, 1, 13, 196], 200),
    "gaussian-g5": ([300, 0, 1], 301),
    "llama-qjl": ([64, 0], 100),
    "sinks-max": ([0, 0, 1, 572], 1024),  # the largest sink count and window capacity together
    "blk-edges": ([0, 1, 16, 0, 31, 1, 17, 48, 100, 1000], 1024),
    "blk-g1-sinks": ([680, 0, 1, 0], 700),
    "blk32-edges": ([1, 0, 16, 1, 0, 47, 300, 1024, 1024], 1024),
}


@pytest.mark.parametrize("name", list(WINDOWS))
def test_decode_attention_hot_window(cases, name):
    c = get(cases, name)
    fmt = c.fmt()
    lens_w, cap = WINDOWS[name]
    print(f"[parity] decode with hot window {name}: lens={c.lens.tolist()} windows={lens_w} cap={cap}",
          flush=True)
    wk, wv, wl_ = c.window(lens_w, cap)
    want = c.oracle_decode_window(wk, wv, wl_)
    got = c.gpu_decode_window(fmt, c.ref_pages_on_gpu(), wk, wv, wl_)
    check_attention(got, want)
    # a window of length 0 everywhere is the plain decode
    if name == "llama-small":
        z = np.zeros_like(wl_)
        plain, _ = c.gpu_decode(fmt, c.ref_pages_on_gpu())
        none = c.gpu_decode_window(fmt, c.ref_pages_on_gpu(), wk, wv, z)
        assert np.array_equal(plain.view(np.uint32), none.view(np.uint32))


def test_decode_explicit_scale(cases):
    c = get(cases, "llama-small")
    fmt = c.fmt()
    got, _ = c.gpu_decode(fmt, c.ref_pages_on_gpu(), scale=0.05)
    check_attention(got, c.oracle_decode(scale=0.05))


def test_quantize_zero_rows_and_skipped_slots():
    import torch
    import packed_decode_attention_amd as tq
    from _parity import oracle_codebooks
    from oracle import quantize as oq
    D, H, kb, vb = 128, 2, 4, 3
    (kc, kt), (vc, vt) = oracle_codebooks(D, kb, vb)
    fmt = tq.LayerFormat(D, H, H, kb, vb, 16, 0, k_codebook=(kc, kt), v_codebook=(vc, vt))
    g = torch.Generator().manual_seed(5)
    k = torch.randn((40, H, D), generator=g).to(torch.float16)
    v = torch.randn((40, H, D), generator=g).to(torch.float16)
    k[3] = 0
    v[7, 1] = 0
    k[9, 0, 5] = 1e-7  # an fp16 subnormal-only row part
    slots = np.random.default_rng(1).permutation(64)[:40].astype(np.int64)
    slots[[2, 11]] = -1
    pages = torch.full((4, 16, H, fmt.slot_stride), 0x77, dtype=torch.uint8, device="cuda")
    tq.tq_quantize_append(fmt.desc, k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), pages, 4)
    torch.cuda.synchronize()
    ref = np.full(4 * 16 * H * fmt.slot_stride, 0x77, np.uint8)
    kt_, vt_ = oq.append_rows_fast(ref, k.numpy(), v.numpy(), slots, kt, vt, kb, vb, 0)
    got = pages.cpu().numpy().reshape(-1)
    compare_pages(got, ref, slots, H, D, kb, vb, fmt.slot_stride, kt_, vt_)
    unwritten = np.setdiff1d(np.arange(64), slots[slots >= 0])
    assert np.all(got.reshape(-1, H, fmt.slot_stride)[unwritten] == 0x77)
    row = got.reshape(-1, H, fmt.slot_stride)[slots[3], 0]
    assert bytes(row[:68]) == bytes([0x88] * 64) + bytes(4)     # zero K row: all indices L/2, norm 0


def test_determinism_repeat_quantize():
    c = _case("ragged-small")
    fmt = c.fmt()
    a = c.gpu_quantize(fmt).cpu().numpy()
    b = c.gpu_quantize(fmt).cpu().numpy()
    assert np.array_equal(a, b)
