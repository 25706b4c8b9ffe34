"""The decode step's calls captured in a HIP graph (torch.cuda.CUDAGraph, through the C ABI): a
serving loop replays one graph per step instead of launching every kernel from the host.

The entry points launch only kernels on the caller's stream (no allocation, fill or host
synchronisation inside a call), so a capture records the same kernels the eager call runs.  Each
case runs the step eagerly on a copy of the pages, captures it on another copy, and replays the
graph three times; between replays the program does eager work of its own (another decode into
another buffer, a fill of the graph's output with NaN) and synchronises.  After every replay the
graph's pages (every byte) and output must equal the eager step's bit for bit.

Cases: the Qwen2.5-0.5B-shaped format (split kernel and merge after a separate append), the
Llama-3-8B-shaped format with the append inside the decode call (block kernel), and a
Mistral-7B-shaped K8/V4 layer with fp16 sinks (sink chunks, split kernel, merge).
"""

import numpy as np
import pytest

from packed_decode_attention_amd import workloads as wl

from _parity import Case

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
CASES = [
    ("qwen-two-calls", wl.scaled(W["qwen2.5-0.5b"], num_seqs=3), [700, 1, 257], False),
    ("llama-fused", wl.scaled(W["llama3-8b"], num_seqs=4), [500, 33, 16, 900], True),
    ("mistral-sinks", wl.scaled(W["mistral-7b"], num_seqs=2), [600, 3], False),
]


@pytest.mark.parametrize("name,w,lens,fused", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_the_eager_step(name, w, lens, fused):
    import torch
    import packed_decode_attention_amd as tq

    print(f"[graph] case {name}: lengths {lens}, fused append {fused}", flush=True)
    c = Case(w, lens=lens)
    fmt = c.fmt()
    L = c.lens
    B, H, D = len(L), c.H, c.D
    last = np.cumsum(L) - 1  # every sequence is non-empty: its last row is the step's new token
    ctx = np.setdiff1d(np.arange(len(c.slots)), last)
    base = torch.full((c.num_blocks, w.block_size, H, c.slot_stride), 0x5A, dtype=torch.uint8, device="cuda")
    tq.tq_quantize_append(fmt.desc, c.k[ctx].cuda(), c.v[ctx].cuda(), torch.from_numpy(c.slots[ctx]).cuda(),
                          base, c.num_blocks)
    q, bt, sl = c.q.cuda(), torch.from_numpy(c.bt).cuda(), torch.from_numpy(L).cuda()
    k_new, v_new = c.k[last].cuda(), c.v[last].cuda()
    new_slots = torch.from_numpy(c.slots[last]).cuda()
    sk = None if c.sink_k is None else c.sink_k.cuda()
    sv = None if c.sink_v is None else c.sink_v.cuda()
    max_len = int(L.max())

    def step(pages, out, ws):
        if fused:
            tq.tq_paged_decode_attention_append(fmt.desc, q, k_new, v_new, pages, c.num_blocks, bt, sl,
                                                max_len, out, ws)
        else:
            tq.tq_quantize_append(fmt.desc, k_new, v_new, new_slots, pages, c.num_blocks)
            tq.tq_paged_decode_attention(fmt.desc, q, pages, c.num_blocks, bt, sl, max_len, out, ws,
                                         sk, sv, w.n_sink)

    pages_e = base.clone()
    out_e = torch.full((B, c.Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    step(pages_e, out_e, fmt.new_workspace(B, max_len))
    torch.cuda.synchronize()
    assert torch.isfinite(out_e).all(), name

    pages_g = base.clone()
    out_g = torch.full_like(out_e, float("nan"))
    ws_g = fmt.new_workspace(B, max_len)
    other_out = torch.empty_like(out_e)
    other_ws = fmt.new_workspace(B, max_len)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(pages_g, out_g, ws_g)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[graph] case {name}: replay {rep}", flush=True)
        out_g.fill_(float("nan"))
        tq.tq_paged_decode_attention(fmt.desc, q, pages_e, c.num_blocks, bt, sl, max_len, other_out,
                                     other_ws, sk, sv, w.n_sink)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(pages_g, pages_e), (name, rep)
        assert torch.equal(out_g.view(torch.int32), out_e.view(torch.int32)), (name, rep)
        assert torch.equal(other_out.view(torch.int32), out_e.view(torch.int32)), (name, rep)
