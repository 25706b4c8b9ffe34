"""tq_paged_decode_attention_noalloc (the decode for callers that cannot allocate: its split-K
partials live in the library's static per-GPU array) against tq_paged_decode_attention with a
caller workspace, through the C ABI: the same kernels, so the outputs must be bit-identical, on
two calls in a row (the second on a smaller batch, so it runs over the first call's partials), and
the size limit is reported as its own error."""

import numpy as np
import pytest

from packed_decode_attention_amd import workloads as wl

from _parity import Case, check_attention

pytestmark = pytest.mark.gpu


def _run_both(c, lens=None):
    import torch
    import packed_decode_attention_amd as tq
    fmt = c.fmt()
    lens = c.lens if lens is None else np.asarray(lens, np.int32)
    B = len(lens)
    max_len = int(lens.max())
    q = c.q[:B].cuda()
    pages = c.ref_pages_on_gpu()
    bt = torch.from_numpy(np.ascontiguousarray(c.bt[:B])).cuda()
    sl = torch.from_numpy(lens).cuda()
    sk = None if c.sink_k is None else c.sink_k[:B].contiguous().cuda()
    sv = None if c.sink_v is None else c.sink_v[:B].contiguous().cuda()
    ws = fmt.new_workspace(B, max_len)
    ref = torch.full((B, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    tq.tq_paged_decode_attention(fmt.desc, q, pages, c.num_blocks, bt, sl, max_len, ref, ws, sk, sv,
                                 c.w.n_sink)
    tq.tq_paged_decode_attention_noalloc(fmt.desc, q, pages, c.num_blocks, bt, sl, max_len, got, sk, sv,
                                         c.w.n_sink)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


CASES = [
    ("llama-g4", dict(w=wl.scaled(wl.WORKLOADS["llama3-8b"], num_seqs=3), lens=[1500, 777, 40])),
    ("mistral-sinks", dict(w=wl.scaled(wl.WORKLOADS["mistral-7b"], num_seqs=3), lens=[900, 3, 130])),
    ("ragged-g8", dict(w=wl.scaled(wl.WORKLOADS["ragged"], num_seqs=4), lens=[613, 64, 1, 300])),
    # the matrix-core split kernel at D = 64, eight bits (the Qwen2.5-0.5B shape)
    ("qwen-d64", dict(w=wl.scaled(wl.WORKLOADS["qwen2.5-0.5b"], num_seqs=3), lens=[4097, 1, 600])),
]


@pytest.mark.parametrize("name,spec", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_call_twice(name, spec):
    spec = dict(spec)
    c = Case(spec.pop("w"), **spec)
    print(f"[no-alloc] {name}: lens={c.lens.tolist()}", flush=True)
    ref, got = _run_both(c)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    check_attention(got, c.oracle_decode())
    # a second call with a smaller batch and shorter sequences: the array still holds the first
    # call's partials, which must not leak into this one
    small = [max(1, int(L) // 3) for L in c.lens[:-1]]
    print(f"[no-alloc] {name}: second call lens={small}", flush=True)
    ref2, got2 = _run_both(c, small)
    assert np.array_equal(ref2.view(np.uint32), got2.view(np.uint32))
    from oracle import attention as oatt
    B2 = len(small)
    sk = None if c.sink_k is None else c.sink_k.numpy()[:B2]
    sv = None if c.sink_v is None else c.sink_v.numpy()[:B2]
    want2 = oatt.decode_attention(c.q.numpy()[:B2], c.pages_ref, c.bt[:B2], np.asarray(small), c.layer_dict,
                                  c.kcb[0], c.vcb[0], sk, sv, c.w.n_sink)
    check_attention(got2, want2)


def test_noalloc_rejects_sizes_beyond_its_array():
    import torch
    import packed_decode_attention_amd as tq
    from packed_decode_attention_amd import _lib
    fmt = tq.LayerFormat(128, 64, 8, 3, 2)
    B, L = 2048, 16384  # 2048 x 8 kv heads x 8 query heads of partials: beyond the static array
    q = torch.zeros((B, 64, 128), dtype=torch.float16, device="cuda")
    out = torch.empty((B, 64, 128), dtype=torch.float32, device="cuda")
    pages = torch.zeros((1, 16, 8, fmt.slot_stride), dtype=torch.uint8, device="cuda")
    bt = torch.zeros((B, L // 16), dtype=torch.int32, device="cuda")
    sl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    assert tq.tq_decode_workspace_bytes(fmt.desc, B, L) > _lib.TQ_NOALLOC_WORKSPACE_BYTES
    with pytest.raises(tq.TqError) as e:
        tq.tq_paged_decode_attention_noalloc(fmt.desc, q, pages, 1, bt, sl, L, out)
    assert e.value.status == _lib.TQ_ERR_NOALLOC_LIMIT


def test_noalloc_accepts_the_full_ragged_batch():
    """The largest benchmark batch (256 sequences of up to 16 385 + 256 tokens, K3/V2, eight query
    heads per kv head) fits the static array; with every length 0 nothing is read and the output
    is zero."""
    import torch
    import packed_decode_attention_amd as tq
    fmt = tq.LayerFormat(128, 64, 8, 3, 2)
    B, L = 256, 16385 + 256
    print(f"[noalloc] full ragged batch sizes: B={B} L={L}", flush=True)
    q = torch.zeros((B, 64, 128), dtype=torch.float16, device="cuda")
    out = torch.full((B, 64, 128), 7.0, dtype=torch.float32, device="cuda")
    pages = torch.zeros((1, 16, 8, fmt.slot_stride), dtype=torch.uint8, device="cuda")
    bt = torch.zeros((B, (L + 15) // 16), dtype=torch.int32, device="cuda")
    sl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    tq.tq_paged_decode_attention_noalloc(fmt.desc, q, pages, 1, bt, sl, L, out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
