"""GPU parity of tq_paged_decode_attention_append (one decode step's append and attention in one
call) through the C ABI.

Each case quantizes every cached position but the last of each sequence with tq_quantize_append,
then runs the step two ways on copies of those pages:
  * tq_quantize_append of the last positions' rows at their slots, then tq_paged_decode_attention;
  * tq_paged_decode_attention_append with the same rows.
Pages (every byte, the untouched slots' 0x5A filler included) and outputs must be identical bit
for bit, and both must match the CPU oracle: packed bytes at the pages' parity bar (identical
apart from listed decision ties), and attention within the tolerance of the other decode tests
against the oracle's decode of the same pages (as the decode parity tests take the oracle's own
pages: an index chosen the other way at a tie moves a 3-bit centroid far enough to show in the
output).

The cases cover both forms of the block kernel's plan (aligned pieces of a uniform batch; ranges
of a ragged one, where one workgroup appends the tokens of many short sequences over several
tiles), new tokens at the first and last position of a 16-position run, an empty sequence, both
block-kernel formats (K4/V4 with four query heads per kv head, K3/V2 with four or eight) and a
block size of 32.
"""

import numpy as np
import pytest

from packed_decode_attention_amd import workloads as wl

from _parity import Case, check_attention, compare_pages
from oracle import attention as oatt

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(2024)
CASES = [
    # uniform batch: aligned pieces, the last piece's workgroup appends its sequence's token
    ("k4v4-aligned", wl.Workload("append-a", 1, 16, 32, 8, 128, 4, 4, 0, values="outliers", seed=41),
     [700] * 16),
    # new tokens at positions 0, 15, 16, 31, 32 of their runs, and an empty sequence
    ("k4v4-run-edges", wl.Workload("append-b", 1, 7, 32, 8, 128, 4, 4, 0, seed=42),
     [1, 16, 17, 32, 33, 0, 500]),
    # ragged lengths, fragmented tables, eight query heads per kv head: the range plan
    ("k3v2-g8-ragged", wl.Workload("append-c", 1, 40, 64, 8, 128, 3, 2, 0, tables="fragmented", seed=43),
     [int(x) for x in _rng.integers(1, 3000, 40)]),
    # 300 short sequences: one workgroup appends the tokens of a dozen or more, over several tiles
    ("k3v2-g4-short", wl.Workload("append-d", 1, 300, 32, 8, 128, 3, 2, 0, seed=44),
     [int(x) for x in _rng.integers(1, 41, 300)]),
    # page blocks of 32 positions
    ("k4v4-bs32", wl.Workload("append-e", 1, 5, 32, 8, 128, 4, 4, 0, block_size=32, seed=45),
     [100, 33, 64, 1, 257]),
    # formats of the matrix-core split kernel, whose last split per (sequence, kv head) appends:
    # the Qwen2.5-0.5B shape (D = 64, K8/V8, 7 query heads per kv head), a new token alone in its
    # split (lengths one past a multiple of the split) and at the first and last rows of a run
    ("split-d64-k8v8", wl.scaled(wl.WORKLOADS["qwen2.5-0.5b"], num_seqs=6), [4097, 1, 16, 17, 300, 0]),
    # K8/V4 at D = 128 with four query heads per kv head (the Mistral-7B layers' format)
    ("split-k8v4", wl.Workload("append-f", 1, 4, 32, 8, 128, 8, 4, 0, values="student_t", seed=47),
     [1000, 2, 513, 32]),
    # K2/V2, four kv heads, page blocks of 32 positions
    ("split-k2v2-bs32", wl.Workload("append-g", 1, 5, 16, 4, 128, 2, 2, 0, block_size=32,
                                    tables="fragmented", seed=48), [64, 65, 1, 900, 31]),
]
# padded slots (a stride of 160 bytes): the append zeroes the padding as the quantizer does
PADDED = [("split-k4v4-pad160", wl.Workload("append-h", 1, 3, 8, 2, 128, 4, 4, 0, seed=49), [300, 45, 1], 160)]


@pytest.mark.parametrize("name,w,lens,stride", [c + (0,) for c in CASES] + PADDED,
                         ids=[c[0] for c in CASES + PADDED])
def test_fused_append_matches_two_calls_and_oracle(name, w, lens, stride):
    import torch
    import packed_decode_attention_amd as tq

    print(f"[append] case {name}: {len(lens)} sequences, lengths {min(lens)}..{max(lens)}", flush=True)
    c = Case(w, lens=lens, slot_stride=stride)
    fmt = c.fmt()
    kernel = tq.decode_kernel_names(c.D, c.kb, c.vb, num_kv_heads=c.H, group=c.Hq // c.H)[0]
    assert kernel == ("tq_decode_mfma_kernel" if name.startswith("split") else "tq_decode_block_kernel")
    L = c.lens
    B, H, D = len(L), c.H, c.D
    last = (np.cumsum(L) - 1)[L > 0]  # row index of each sequence's new token
    ctx = np.setdiff1d(np.arange(len(c.slots)), last)
    base = torch.full((c.num_blocks, w.block_size, H, c.slot_stride), 0x5A, dtype=torch.uint8, device="cuda")
    tq.tq_quantize_append(fmt.desc, c.k[ctx].cuda(), c.v[ctx].cuda(), torch.from_numpy(c.slots[ctx]).cuda(),
                          base, c.num_blocks)
    k_new = torch.zeros(B, H, D, dtype=torch.float16)
    v_new = torch.zeros(B, H, D, dtype=torch.float16)
    k_new[torch.from_numpy(L > 0)] = c.k[last]
    v_new[torch.from_numpy(L > 0)] = c.v[last]
    q, bt, sl = c.q.cuda(), torch.from_numpy(c.bt).cuda(), torch.from_numpy(L).cuda()
    max_len = int(L.max())

    pages_two = base.clone()
    out_two = torch.full((B, c.Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_quantize_append(fmt.desc, c.k[last].cuda(), c.v[last].cuda(), torch.from_numpy(c.slots[last]).cuda(),
                          pages_two, c.num_blocks)
    tq.tq_paged_decode_attention(fmt.desc, q, pages_two, c.num_blocks, bt, sl, max_len, out_two,
                                 fmt.new_workspace(B, max_len))

    pages_one = base.clone()
    out_one = torch.full((B, c.Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_paged_decode_attention_append(fmt.desc, q, k_new.cuda(), v_new.cuda(), pages_one, c.num_blocks,
                                        bt, sl, max_len, out_one, fmt.new_workspace(B, max_len))
    torch.cuda.synchronize()

    assert torch.equal(pages_one, pages_two), name
    assert torch.equal(out_one.view(torch.int32), out_two.view(torch.int32)), name
    got_pages = pages_one.cpu().numpy().reshape(-1)
    compare_pages(got_pages, c.pages_ref, c.slots, H, D, c.kb, c.vb, c.slot_stride, c.k_tie, c.v_tie)
    want = oatt.decode_attention(c.q.numpy(), got_pages, c.bt, c.lens, c.layer_dict, c.kcb[0], c.vcb[0],
                                 None, None, 0)
    check_attention(out_one.cpu().numpy(), want)


def test_fused_append_repeated_steps():
    """Three steps in a row on the same pages, each appending one more token per sequence (the
    serving loop's pattern), against the two-call path step by step."""
    import torch
    import packed_decode_attention_amd as tq

    w = wl.Workload("append-steps", 1, 24, 64, 8, 128, 3, 2, 0, tables="fragmented", seed=46)
    lens = np.array([int(x) for x in np.random.default_rng(7).integers(20, 900, 24)], np.int32)
    c = Case(w, lens=lens + 3)  # rows for three more steps
    fmt = c.fmt()
    B, H, D = len(lens), c.H, c.D
    starts = np.cumsum(c.lens) - c.lens
    ctx = np.concatenate([starts[b] + np.arange(lens[b]) for b in range(B)])
    pages_one = torch.full((c.num_blocks, w.block_size, H, c.slot_stride), 0x5A, dtype=torch.uint8,
                           device="cuda")
    tq.tq_quantize_append(fmt.desc, c.k[ctx].cuda(), c.v[ctx].cuda(), torch.from_numpy(c.slots[ctx]).cuda(),
                          pages_one, c.num_blocks)
    pages_two = pages_one.clone()
    bt = torch.from_numpy(c.bt).cuda()
    q = c.q.cuda()
    for step in range(3):
        print(f"[append] step {step}", flush=True)
        cur = lens + step + 1
        rows = starts + cur - 1
        sl = torch.from_numpy(cur.astype(np.int32)).cuda()
        out_two = torch.empty((B, c.Hq, D), dtype=torch.float32, device="cuda")
        out_one = torch.empty_like(out_two)
        tq.tq_quantize_append(fmt.desc, c.k[rows].cuda(), c.v[rows].cuda(),
                              torch.from_numpy(c.slots[rows]).cuda(), pages_two, c.num_blocks)
        tq.tq_paged_decode_attention(fmt.desc, q, pages_two, c.num_blocks, bt, sl, int(cur.max()), out_two,
                                     fmt.new_workspace(B, int(cur.max())))
        tq.tq_paged_decode_attention_append(fmt.desc, q, c.k[rows].cuda(), c.v[rows].cuda(), pages_one,
                                            c.num_blocks, bt, sl, int(cur.max()), out_one,
                                            fmt.new_workspace(B, int(cur.max())))
        torch.cuda.synchronize()
        assert torch.equal(pages_one, pages_two), step
        assert torch.equal(out_one.view(torch.int32), out_two.view(torch.int32)), step
