"""GPU edge cases of the HIP path through the C ABI, against the CPU oracle:

* sequences made only of fp16 sink tokens, decoded with no page tensor and no block table at all
  (the contract says sink page slots are ignored, and the host accepts NULL for both when no
  sequence is longer than the sinks);
* page slots that no decode may read (the sinks' slots, the hot window's slots, the unwritten
  slots after a sequence's last token) filled with 0xFF bytes, whose norms are NaN: the output
  must be bit-identical to the run on clean pages;
* caller-supplied codebooks whose boundaries are closer than the quantizer's bucket table
  resolves, which send the quantizer down its binary-search decision loop.
"""

import numpy as np
import pytest

from packed_decode_attention_amd import workloads as wl

from _parity import Case, check_attention, compare_pages

pytestmark = pytest.mark.gpu

# (name, workload, lens): the kernels each format reaches are named after the workload
SINK_ONLY = [
    # matrix-core kernel, staged tiles (block size 16), G = 4
    ("k4v4-g4", wl.Workload("sink-only-a", 1, 6, 32, 8, 128, 4, 4, 0, n_sink=8, values="outliers",
                            seed=31), [8, 3, 0, 5, 1, 8]),
    # matrix-core kernel with 8 query heads per kv head (its fp16 rows run as a kernel of their own)
    ("k3v2-g8", wl.Workload("sink-only-b", 1, 3, 64, 8, 128, 3, 2, 0, n_sink=6, seed=32), [6, 2, 4]),
    # matrix-core kernel, per-lane fetch (block size 7), D = 64
    ("k8v8-d64-bs7", wl.Workload("sink-only-c", 1, 3, 10, 2, 64, 8, 8, 0, block_size=7, n_sink=9,
                                 seed=33), [9, 7, 1]),
    # vector kernel (3-bit values)
    ("k2v3-vector", wl.Workload("sink-only-d", 1, 3, 6, 2, 128, 2, 3, 0, n_sink=4, seed=34), [4, 2, 3]),
]


@pytest.mark.parametrize("name,w,lens", SINK_ONLY, ids=[s[0] for s in SINK_ONLY])
def test_decode_sink_only_sequences_without_pages(name, w, lens):
    import torch
    import packed_decode_attention_amd as tq
    c = Case(w, lens=lens)
    fmt = c.fmt()
    B = len(lens)
    max_len = max(lens)
    assert max_len <= w.n_sink
    print(f"[edges] sink-only {name}: lens={lens} n_sink={w.n_sink}, no pages, no block table", flush=True)
    out = torch.full((B, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
    ws = fmt.new_workspace(B, max_len)
    tq.tq_paged_decode_attention(fmt.desc, c.q.cuda(), None, 0, None, torch.from_numpy(c.lens).cuda(),
                                 max_len, out, ws, c.sink_k.cuda(), c.sink_v.cuda(), w.n_sink)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    check_attention(got, c.oracle_decode())
    assert np.all(got[c.lens == 0] == 0)


def _dirty_pages(c, win_lens=None):
    """The oracle's pages with every slot a decode must not read set to 0xFF: the sinks' slots,
    the hot window's slots and the unwritten slots after each sequence's last token."""
    pages = c.pages_ref.reshape(-1, c.H, c.slot_stride).copy()
    bs = c.w.block_size
    for b, L in enumerate(c.lens):
        L = int(L)
        nblk = (max(L, 1) + bs - 1) // bs
        ns = min(c.w.n_sink, L)
        w = 0 if win_lens is None else int(win_lens[b])
        pos = np.concatenate([np.arange(ns), np.arange(L - w, L), np.arange(L, nblk * bs)]).astype(np.int64)
        slots = wl.token_slots(c.bt, b, pos, bs)
        pages[slots] = 0xFF
    return pages.reshape(-1)


DIRTY = [
    # staged matrix-core tiles, G = 4; 20 sinks put the first packed run mid-block (positions 16..19
    # of that run are sink slots)
    ("k4v4-g4", dict(w=wl.Workload("dirty-a", 1, 4, 32, 8, 128, 4, 4, 0, n_sink=20, values="outliers",
                                   seed=41), lens=[700, 33, 20, 21]), [64, 13, 0, 1]),
    # staged tiles of the mean-removal format
    ("k4v4-mean", dict(w=wl.Workload("dirty-b", 1, 3, 32, 8, 128, 4, 4, 0, n_sink=5, seed=42),
                       lens=[300, 37, 6], mean_removal=True), [17, 32, 1]),
    # 8 query heads per kv head, 3-bit keys
    ("k3v2-g8", dict(w=wl.Workload("dirty-c", 1, 3, 64, 8, 128, 3, 2, 0, n_sink=4, seed=43),
                     lens=[400, 5, 77]), [100, 1, 0]),
    # per-lane fetch (block size 7), D = 64, 8-bit codes
    ("k8v8-d64-bs7", dict(w=wl.Workload("dirty-d", 1, 3, 10, 2, 64, 8, 8, 0, block_size=7, n_sink=9,
                                        seed=44), lens=[200, 10, 9]), [20, 1, 0]),
    # the QJL key format on the matrix cores
    ("k4v4-qjl", dict(w=wl.Workload("dirty-e", 1, 2, 32, 8, 128, 4, 4, 0, n_sink=3, seed=45),
                      lens=[150, 40], qjl=True), [9, 3]),
    # vector kernel (3-bit values), block size 7
    ("k2v3-vector", dict(w=wl.Workload("dirty-f", 1, 3, 6, 2, 128, 2, 3, 0, block_size=7, n_sink=4,
                                       seed=46), lens=[90, 5, 4]), [11, 1, 0]),
]


@pytest.mark.parametrize("name,spec,win", DIRTY, ids=[d[0] for d in DIRTY])
def test_decode_ignores_slots_outside_the_packed_range(name, spec, win):
    import torch
    spec = dict(spec)
    c = Case(spec.pop("w"), **spec)
    fmt = c.fmt()
    print(f"[edges] 0xFF slots {name}: lens={c.lens.tolist()} n_sink={c.w.n_sink} windows={win}", flush=True)
    clean = c.ref_pages_on_gpu()
    dirty = torch.from_numpy(_dirty_pages(c)).cuda().reshape(clean.shape)
    want = c.oracle_decode()
    got_clean, _ = c.gpu_decode(fmt, clean)
    got_dirty, _ = c.gpu_decode(fmt, dirty)
    check_attention(got_dirty, want)
    assert np.array_equal(got_clean.view(np.uint32), got_dirty.view(np.uint32))
    if c.qjl:
        return  # the hot window is a separate call; once per kernel family is enough
    # with a hot window: its slots are dirty too
    cap = max(win) + 3
    wk, wv, wl_ = c.window(win, cap)
    dirty_w = torch.from_numpy(_dirty_pages(c, wl_)).cuda().reshape(clean.shape)
    ref = c.oracle_decode_window(wk, wv, wl_)
    a = c.gpu_decode_window(fmt, clean, wk, wv, wl_)
    b = c.gpu_decode_window(fmt, dirty_w, wk, wv, wl_)
    check_attention(b, ref)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _tight_codebook(D, bits, gap_exp):
    """The oracle's Beta codebook with the boundary above the middle one (which is 0) moved to
    2^gap_exp, where the rotated coordinates are densest; centroids left as they are: decisions
    depend on the boundaries only."""
    from oracle import codebook as ocb
    cb = ocb.codebook(D, bits)
    t = cb.boundaries32.astype(np.float64).copy()
    k = len(t) // 2 + 1
    assert t[k - 1] == 0.0
    t[k] = t[k - 1] + 2.0 ** gap_exp
    assert t[k] < t[k + 1]
    t32 = t.astype(np.float32)
    assert np.min(np.diff(t32.astype(np.float64))) <= 2.0 ** gap_exp
    return cb.centroids32, t32


@pytest.mark.parametrize("D,kb,vb,gap_exp", [(128, 8, 4, -12), (128, 4, 3, -7), (64, 4, 8, -8)])
def test_quantize_fine_codebooks_take_the_search_loop(D, kb, vb, gap_exp):
    """A boundary gap finer than the bucket table resolves (2^-12 at 8 bits, under 2^-6 at 4 bits)
    sends both regions of every tile to the binary search; the bytes must still equal the oracle's
    decisions on those boundaries."""
    import torch
    import packed_decode_attention_amd as tq
    from oracle import quantize as oq
    H, n_tok, bs = 4, 1500, 16
    from oracle import codebook as ocb
    kc, kt = _tight_codebook(D, kb, gap_exp)
    vcb = ocb.codebook(D, vb)  # a plain V codebook: the search loop serves both regions anyway
    vc, vt = vcb.centroids32, vcb.boundaries32
    fmt = tq.LayerFormat(D, H, H, kb, vb, bs, 0, k_codebook=(kc, kt), v_codebook=(vc, vt))
    g = torch.Generator().manual_seed(100 + kb)
    k = torch.randn((n_tok, H, D), generator=g).to(torch.float16)
    v = (torch.randn((n_tok, H, D), generator=g) * 3).to(torch.float16)
    nblk = (n_tok + bs - 1) // bs + 2
    slots = np.random.default_rng(kb).permutation(nblk * bs)[:n_tok].astype(np.int64)
    slots[[5, 700]] = -1
    print(f"[edges] search loop D={D} K{kb}/V{vb} gap 2^{gap_exp}: {n_tok} tokens x {H} heads", flush=True)
    pages = torch.full((nblk, bs, H, fmt.slot_stride), 0x33, dtype=torch.uint8, device="cuda")
    tq.tq_quantize_append(fmt.desc, k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), pages, nblk)
    torch.cuda.synchronize()
    ref = np.full(nblk * bs * H * fmt.slot_stride, 0x33, np.uint8)
    k_tie, v_tie = oq.append_rows_fast(ref, k.numpy(), v.numpy(), slots, kt, vt, kb, vb, 0)
    ties = compare_pages(pages.cpu().numpy().reshape(-1), ref, slots, H, D, kb, vb, fmt.slot_stride,
                         k_tie, v_tie)
    assert ties <= max(4, 1e-4 * n_tok * H * D)
    # the moved boundary is exercised: some coordinates fall between the two close boundaries
    u = oq.rotated_unit(k.numpy(), 0)
    k_mid = len(kt) // 2 + 1
    assert np.any((u >= kt[k_mid - 1]) & (u < kt[k_mid]))
