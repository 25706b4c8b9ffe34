"""Parity at the benchmark's full sizes, in the launch configuration bench.py times.

Each case fills one layer of a full-size workload exactly as the benchmark does (bulk
quantize-append of the whole context in chunks, then the decode step's one-token append), then runs
decode over the whole batch.  A few sampled (sequence, kv head) pairs are recomputed by the CPU
oracle from the same fp16 rows:
  * their packed page rows must equal the oracle's (indices at listed ties excepted);
  * with the oracle's bytes written into their page rows (so ties cannot move a key), the decode
    output of the query heads of that kv head must match the oracle's dense attention to the
    attention tolerance.
The rest of the batch still runs, so the grid, split geometry and workspace are the benchmark's.
One case uses the norm-correction page format (bench.py --norm-correction), one the mean-removal
format (bench.py --mean-removal), one the QJL key format (bench.py --qjl), one decodes two
causal queries per sequence (bench.py --queries 2).  One case adds a hot
window (bench.py --hot-window): the last W positions of every sequence also
come from fp16 rows (the sampled sequences' own rows, random rows elsewhere) and the decode runs
through tq_paged_decode_attention_window.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest

from _parity import check_attention, compare_pages, oracle_codebooks
from oracle import attention as oatt
from oracle import quantize as oq

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def _pick(w, lens, which):
    if which == "extremes":
        return [int(np.argmax(lens)), int(np.argmin(lens))]
    return list(which)


CASES = [  # workload, layer, sampled sequences, hot window, format (True: norm correction), queries
    ("llama3-8b", 1, (0, 13), 0, False, 1),
    ("mistral-7b", 2, (1,), 0, False, 1),
    ("ragged", 5, "extremes", 0, False, 1),
    ("qwen2.5-0.5b", 7, (0, 5), 0, False, 1),
    ("llama3-8b", 3, (4,), 512, False, 1),
    ("llama3-8b", 6, (9,), 0, True, 1),
    ("llama3-8b", 2, (3,), 0, False, 2),
    ("llama3-8b", 5, (7,), 0, "mean", 1),
    ("llama3-8b", 4, (11,), 0, "qjl", 1),
]


@pytest.mark.parametrize("name,layer,which,window,nc,nq", CASES,
                         ids=[f"{c[0]}-L{c[1]}" + (f"-W{c[3]}" if c[3] else "")
                              + ("-MEAN" if c[4] == "mean" else "-QJL" if c[4] == "qjl" else
                                 "-NC" if c[4] else "")
                              + (f"-Q{c[5]}" if c[5] > 1 else "") for c in CASES])
def test_full_size_sampled(name, layer, which, window, nc, nq):
    import torch
    import packed_decode_attention_amd as tq
    from packed_decode_attention_amd import workloads as wl
    bench = _bench()

    w = wl.WORKLOADS[name]
    kb, vb = w.bits(layer)
    B, H, D, Hq, bs = w.num_seqs, w.num_kv_heads, w.head_dim, w.num_q_heads, w.block_size
    lens = wl.seq_lens(w)
    bt_np, num_blocks = wl.block_tables(w, lens)
    ctx_np, new_np = bench.context_slots(w, bt_np, lens, wl)
    seqs = _pick(w, lens, which)
    print(f"[fullsize] {name} layer {layer} K{kb}/V{vb}: B={B} max_len={int(lens.max())} "
          f"sampled sequences {seqs}", flush=True)

    heads = {b: (7 * b + layer) % H for b in seqs}  # one kv head per sampled sequence
    G = Hq // H
    mean = nc == "mean"  # the format column: norm correction, mean removal or the QJL key sketch
    qjl = nc == "qjl"
    nc = nc is True
    fmt = tq.LayerFormat(D, Hq, H, kb, vb, bs, 0, norm_correction=nc, mean_removal=mean, qjl=qjl)
    pages = fmt.new_pages(num_blocks)
    ctx_off = np.concatenate([[0], np.cumsum(lens - 1)])
    rows = {b: ([], []) for b in seqs}

    def tap(s0, k, v):
        n = k.shape[0]
        for b in seqs:
            lo, hi = max(int(ctx_off[b]), s0), min(int(ctx_off[b + 1]), s0 + n)
            if lo < hi:
                hh = heads[b]
                rows[b][0].append(k[lo - s0:hi - s0, hh:hh + 1].cpu())
                rows[b][1].append(v[lo - s0:hi - s0, hh:hh + 1].cpu())

    bench.fill_layer(w, layer, fmt, pages, torch.from_numpy(ctx_np).cuda(), num_blocks, torch, tq, wl,
                     tap=tap)
    new_k, new_v = bench.new_tokens(w, 1, wl)
    new_slots = torch.from_numpy(new_np).cuda()
    tq.tq_quantize_append(fmt.desc, new_k[0, layer], new_v[0, layer], new_slots, pages, num_blocks)
    torch.cuda.synchronize()

    (kc, kt), (vc, vt) = oracle_codebooks(D, kb, vb)
    stride = fmt.slot_stride
    flat = pages.view(-1, H, stride)
    refs = {}
    for b in seqs:
        L, hh = int(lens[b]), heads[b]
        k = torch.cat(rows[b][0] + [new_k[0, layer, b:b + 1, hh:hh + 1].cpu()]).numpy()
        v = torch.cat(rows[b][1] + [new_v[0, layer, b:b + 1, hh:hh + 1].cpu()]).numpy()
        assert k.shape == (L, 1, D)
        # oracle pages of this one (sequence, kv head), identity table
        one = wl.scaled(w, num_seqs=1, tables="identity")
        bt1, nblk1 = wl.block_tables(one, np.array([L]))
        slots1 = wl.token_slots(bt1, 0, np.arange(L), bs)
        ref = np.zeros(nblk1 * bs * stride, np.uint8)
        cents = dict(k_centroids32=kc, v_centroids32=vc) if nc else {}
        ties_ = oq.append_rows_fast(ref, k, v, slots1, kt, vt, kb, vb, 0, stride, mean=mean,
                                    qjl_centroids32=kc if qjl else None, **cents)
        k_tie, v_tie, q_tie = ties_ if qjl else ties_ + (None,)
        # the GPU's rows of the same positions and kv head
        slots = torch.from_numpy(wl.token_slots(bt_np, b, np.arange(L), bs)).cuda()
        gpu_rows = flat[slots, hh].cpu().numpy()
        ref_rows = ref.reshape(-1, stride)[slots1]
        nc_args = ((oq.norm_fp32(k), oq.norm_fp32(v)), (kc, vc)) if nc else None
        ties = compare_pages(gpu_rows.reshape(-1), ref_rows.reshape(-1), np.arange(L), 1, D, kb, vb,
                             stride, k_tie, v_tie, nc_args, mean, q_tie)
        print(f"[fullsize]   seq {b} kv head {hh} (L={L}): page rows match, {ties} tie indices",
              flush=True)
        # the oracle's bytes into the GPU pages of this sequence and kv head
        flat[slots, hh] = torch.from_numpy(ref_rows).cuda()
        refs[b] = (ref, bt1, L, k, v)

    q = wl.queries(w, layer, 0, "cuda")
    if nq > 1:  # [B, T, H_q, D]: the queries of the last T positions
        q = torch.stack([wl.queries(w, layer, j, "cuda") for j in range(nq)], dim=1)
    sink_k, sink_v = wl.sinks(w, 0, "cuda")
    max_len = int(lens.max())
    ws = fmt.new_workspace(B, max_len, n_queries=nq if nq > 1 else 0)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device="cuda")
    win_lens = np.minimum(window, lens - np.minimum(lens, w.n_sink)).astype(np.int32)
    if window:
        g = torch.Generator(device="cuda").manual_seed(99)
        win_k = torch.randn((B, window, H, D), generator=g, device="cuda").half()
        win_v = torch.randn((B, window, H, D), generator=g, device="cuda").half()
        for b in seqs:  # the sampled sequences' own last rows, in reverse order
            _, _, L, k, v = refs[b]
            nw = int(win_lens[b])
            win_k[b, :nw, heads[b]] = torch.from_numpy(k[L - nw:L, 0][::-1].copy()).cuda()
            win_v[b, :nw, heads[b]] = torch.from_numpy(v[L - nw:L, 0][::-1].copy()).cuda()
        tq.tq_paged_decode_attention_window(fmt.desc, q, pages, num_blocks, torch.from_numpy(bt_np).cuda(),
                                            torch.from_numpy(lens).cuda(), max_len, out, ws, win_k, win_v,
                                            torch.from_numpy(win_lens).cuda(), sink_k, sink_v, w.n_sink)
    elif nq > 1:
        tq.tq_paged_decode_attention_multi(fmt.desc, q, pages, num_blocks, torch.from_numpy(bt_np).cuda(),
                                           torch.from_numpy(lens).cuda(), max_len, out, ws, sink_k,
                                           sink_v, w.n_sink)
    else:
        tq.tq_paged_decode_attention(fmt.desc, q, pages, num_blocks, torch.from_numpy(bt_np).cuda(),
                                     torch.from_numpy(lens).cuda(), max_len, out, ws, sink_k, sink_v,
                                     w.n_sink)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite output in the batch"
    layer_dict = dict(D=D, H_kv=1, block_size=bs, k_bits=kb, v_bits=vb, seed=0, slot_stride=stride,
                      mean=mean, qjl=qjl)
    qn = q.cpu().numpy()
    skn = None if sink_k is None else sink_k.cpu().numpy()
    svn = None if sink_v is None else sink_v.cpu().numpy()
    for b in seqs:
        ref, bt1, L, k, v = refs[b]
        hh = heads[b]
        qh = slice(hh * G, (hh + 1) * G)  # the query heads that read kv head hh
        nw = int(win_lens[b])
        wkw = dict(win_k16=k[L - nw:L][None], win_v16=v[L - nw:L][None], win_lens=np.array([nw])) if window else {}
        sks = None if skn is None else skn[b:b + 1, :, hh:hh + 1]
        svs = None if svn is None else svn[b:b + 1, :, hh:hh + 1]
        if nq > 1:
            want = oatt.decode_attention_multi(qn[b:b + 1, :, qh], ref, bt1, np.array([L], np.int32),
                                               layer_dict, kc, vc, sks, svs, w.n_sink)
            max_abs, rel = check_attention(got[b:b + 1, :, qh].reshape(nq, G, D), want.reshape(nq, G, D))
        else:
            want = oatt.decode_attention(qn[b:b + 1, qh], ref, bt1, np.array([L], np.int32), layer_dict,
                                         kc, vc, sks, svs, w.n_sink, **wkw)
            max_abs, rel = check_attention(got[b:b + 1, qh], want)
        print(f"[fullsize]   seq {b} kv head {hh}: decode max-abs {max_abs:.2e}, rel L2 {rel:.2e}",
              flush=True)


FUSED = [("llama3-8b", 1), ("ragged", 5), ("qwen2.5-0.5b", 7)]


@pytest.mark.parametrize("name,layer", FUSED, ids=[f"{n}-L{l}" for n, l in FUSED])
def test_full_size_fused_append(name, layer):
    """The benchmark's step at full size: tq_paged_decode_attention_append against
    tq_quantize_append + tq_paged_decode_attention on the same filled layer.  Pages (all of them)
    and outputs must be identical bit for bit; the two-call path is held to the oracle above."""
    import torch
    import packed_decode_attention_amd as tq
    from packed_decode_attention_amd import workloads as wl
    bench = _bench()

    w = wl.WORKLOADS[name]
    kb, vb = w.bits(layer)
    B, H, D, Hq, bs = w.num_seqs, w.num_kv_heads, w.head_dim, w.num_q_heads, w.block_size
    lens = wl.seq_lens(w)
    bt_np, num_blocks = wl.block_tables(w, lens)
    ctx_np, new_np = bench.context_slots(w, bt_np, lens, wl)
    print(f"[fullsize] fused append {name} layer {layer} K{kb}/V{vb}: B={B} max_len={int(lens.max())}",
          flush=True)
    fmt = tq.LayerFormat(D, Hq, H, kb, vb, bs, 0)
    # the block kernel (Llama, ragged) or the matrix-core split kernel's last split (Qwen) appends
    assert tq.decode_kernel_names(D, kb, vb, False, H, Hq // H)[0] in ("tq_decode_block_kernel",
                                                                       "tq_decode_mfma_kernel")
    ctx_pages = fmt.new_pages(num_blocks)
    bench.fill_layer(w, layer, fmt, ctx_pages, torch.from_numpy(ctx_np).cuda(), num_blocks, torch, tq, wl)
    new_k, new_v = bench.new_tokens(w, 1, wl)
    q = wl.queries(w, layer, 0, "cuda")
    bt, sl = torch.from_numpy(bt_np).cuda(), torch.from_numpy(lens).cuda()
    max_len = int(lens.max())

    pages_two = ctx_pages.clone()
    out_two = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_quantize_append(fmt.desc, new_k[0, layer], new_v[0, layer], torch.from_numpy(new_np).cuda(),
                          pages_two, num_blocks)
    tq.tq_paged_decode_attention(fmt.desc, q, pages_two, num_blocks, bt, sl, max_len, out_two,
                                 fmt.new_workspace(B, max_len))
    pages_one = ctx_pages
    out_one = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_paged_decode_attention_append(fmt.desc, q, new_k[0, layer], new_v[0, layer], pages_one,
                                        num_blocks, bt, sl, max_len, out_one, fmt.new_workspace(B, max_len))
    torch.cuda.synchronize()
    assert torch.equal(pages_one, pages_two)
    assert torch.equal(out_one.view(torch.int32), out_two.view(torch.int32))
    print(f"[fullsize]   pages ({pages_one.numel() / 1e6:.0f} MB) and outputs identical", flush=True)
