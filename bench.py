"""Benchmark of the packed-KV decode step on one MI355X.

A step is one pass of the whole hot path over one batch: for every layer, quantize-on-append of
one new token per sequence into the packed pages, then fused paged decode attention over all
cached tokens.  Where the format allows it (the whole-block decode formats, no sinks, window or
extra queries) both run in one call, tq_paged_decode_attention_append; --separate-append times
the two calls instead.  Inputs (pages filled by a bulk quantize of the context, queries, new tokens) are
resident in HBM before timing starts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload llama3-8b] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed-KV decode attention: KV tokens/s + achieved HBM GB/s vs peak, 1 GPU"
HBM_PEAK_GBS = 8000.0
BULK_CHUNK = 1 << 18  # tokens per bulk-fill quantize call


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def describe(w):
    pol = f"K{w.k_bits}/V{w.v_bits}"
    if w.protected:
        pol += " (layers " + ",".join(str(k) for k in sorted(w.protected)) + " K8/V8)"
    ctx = f"{w.context}+1" if w.ragged is None else f"U[{w.ragged[0]},{w.ragged[1]}]+1"
    s = (f"{w.name}: {w.layers} layers, {w.num_seqs} seqs x {ctx} tokens, {w.num_q_heads}/"
         f"{w.num_kv_heads} heads, D={w.head_dim}, {pol} TQ pages bs{w.block_size}")
    if w.n_sink:
        s += f", {w.n_sink} fp16 sinks"
    return s


class LayerState:
    def __init__(self, fmt, pages, num_blocks):
        self.fmt, self.pages, self.num_blocks = fmt, pages, num_blocks
        self.win_k = self.win_v = None  # fp16 hot window [B, W, H_kv, D] (with --hot-window)
        self.fused = False              # append and decode in one call


def context_slots(w, bt_np, lens, wl):
    """Slots of every cached position but the last of each sequence (the bulk-filled context), in
    sequence order, and the slot of each sequence's last position (the decode step's append)."""
    ctx = [wl.token_slots(bt_np, b, np.arange(lens[b] - 1), w.block_size) for b in range(w.num_seqs)]
    new = np.array([wl.token_slots(bt_np, b, [lens[b] - 1], w.block_size)[0] for b in range(w.num_seqs)],
                   np.int64)
    return np.concatenate(ctx), new


def fill_layer(w, l, fmt, pages, ctx_slots, num_blocks, torch, tq, wl, dev="cuda", tap=None):
    """Bulk quantize-append of layer l's context in chunks of BULK_CHUNK tokens; returns the summed
    kernel time in ms.  tap(s0, k, v) sees each chunk's fp16 rows (for parity sampling)."""
    gk = wl.generator(w.seed * 1000003 + l * 31, dev)
    gv = wl.generator(w.seed * 1000003 + l * 31 + 1, dev)
    n_ctx = int(ctx_slots.numel())
    t_layer = 0.0
    for s0 in range(0, n_ctx, BULK_CHUNK):
        n = min(BULK_CHUNK, n_ctx - s0)
        k = wl.kv_values(w, l, n, "k", dev, gen=gk)
        v = wl.kv_values(w, l, n, "v", dev, gen=gv)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tq.tq_quantize_append(fmt.desc, k, v, ctx_slots[s0:s0 + n], pages, num_blocks)
        e1.record()
        e1.synchronize()
        t_layer += e0.elapsed_time(e1)
        if tap is not None:
            tap(s0, k, v)
        del k, v
    return t_layer


def new_tokens(w, n_steps_total, wl, dev="cuda"):
    """fp16 K and V of the token each step appends: [steps, layers, B, H_kv, D] each."""
    B, H, D = w.num_seqs, w.num_kv_heads, w.head_dim
    gnew = wl.generator(w.seed * 99991 + 17, dev)
    new_k = wl.kv_values(w, 0, n_steps_total * w.layers * B, "k", dev, gen=gnew).reshape(
        n_steps_total, w.layers, B, H, D)
    new_v = wl.kv_values(w, 0, n_steps_total * w.layers * B, "v", dev, gen=gnew).reshape(
        n_steps_total, w.layers, B, H, D)
    return new_k, new_v


def setup(w, torch, tq, wl, n_steps_total, hot_window=0, norm_correction=False, n_queries=1,
          mean_removal=False, qjl=False, fused=True):
    lens = wl.seq_lens(w)                       # includes the token appended each step
    bt_np, num_blocks = wl.block_tables(w, lens)
    dev = "cuda"
    bt = torch.from_numpy(bt_np).to(dev)
    seq_lens = torch.from_numpy(lens).to(dev)
    B, H, D = w.num_seqs, w.num_kv_heads, w.head_dim
    ctx_np, new_np = context_slots(w, bt_np, lens, wl)
    ctx_slots = torch.from_numpy(ctx_np).to(dev)
    new_slots = torch.from_numpy(new_np).to(dev)
    fmts = {}
    layers = []
    bulk_ms, bulk_rows = [], 0
    n_ctx = int(ctx_slots.numel())
    for l in range(w.layers):
        kb, vb = w.bits(l)
        if (kb, vb) not in fmts:
            fmts[(kb, vb)] = tq.LayerFormat(D, w.num_q_heads, H, kb, vb, w.block_size, 0,
                                            norm_correction=norm_correction,
                                            mean_removal=mean_removal, qjl=qjl)
        fmt = fmts[(kb, vb)]
        pages = fmt.new_pages(num_blocks)
        t_layer = fill_layer(w, l, fmt, pages, ctx_slots, num_blocks, torch, tq, wl)
        if l > 0:  # layer 0 includes first-launch costs
            bulk_ms.append(t_layer)
        bulk_rows = n_ctx * H
        st = LayerState(fmt, pages, num_blocks)
        st.fused = (fused and fmt.flags == 0 and not hot_window and n_queries == 1 and w.n_sink == 0
                    and B <= tq.TQ_APPEND_MAX_SEQS and w.block_size % 16 == 0 and tq.decode_kernel_names(
                        D, kb, vb, False, H, w.group, 0)[0] in ("tq_decode_block_kernel", "tq_decode_mfma_kernel"))
        if hot_window:  # the last hot_window positions as fp16 rows (their page slots are ignored)
            g = wl.generator(w.seed * 7919 + l, dev)
            shape = (B, hot_window, H, D)
            st.win_k = wl.kv_values(w, l, B * hot_window, "k", dev, gen=g).reshape(shape)
            st.win_v = wl.kv_values(w, l, B * hot_window, "v", dev, gen=g).reshape(shape)
        layers.append(st)
    torch.cuda.synchronize()
    # per-step inputs: queries and one new K/V token per sequence and layer
    if n_queries > 1:  # [B, T, H_q, D]: the queries of the last T positions
        qs = [torch.stack([wl.queries(w, l, j, dev) for j in range(n_queries)], dim=1)
              for l in range(w.layers)]
    else:
        qs = [wl.queries(w, l, 0, dev) for l in range(w.layers)]
    new_k, new_v = new_tokens(w, n_steps_total, wl, dev)
    sink_k, sink_v = wl.sinks(w, 0, dev)
    max_len = int(lens.max())
    nq = n_queries if n_queries > 1 else 0
    ws = fmts[(w.k_bits, w.v_bits)].new_workspace(B, max_len, n_queries=nq)
    for f in fmts.values():
        need = (tq.tq_decode_multi_workspace_bytes(f.desc, B, max_len, n_queries) if nq
                else tq.tq_decode_workspace_bytes(f.desc, B, max_len))
        assert need <= ws.numel()
    out_shape = (B, n_queries, w.num_q_heads, D) if nq else (B, w.num_q_heads, D)
    out = torch.empty(out_shape, dtype=torch.float32, device=dev)
    # several queries: each step appends T rows per sequence, at its last T positions
    multi_slots = None
    if nq:
        multi_slots = torch.from_numpy(np.concatenate(
            [wl.token_slots(bt_np, b, np.arange(lens[b] - n_queries, lens[b]), w.block_size)
             for b in range(B)]).astype(np.int64)).to(dev)
    ns = np.minimum(lens, w.n_sink)
    win_lens = np.minimum(hot_window, lens - ns).astype(np.int32)
    return dict(hot_window=hot_window, win_lens_np=win_lens, win_lens=torch.from_numpy(win_lens).to(dev),
                lens=lens, bt=bt, seq_lens=seq_lens, new_slots=new_slots, layers=layers, qs=qs,
                new_k=new_k, new_v=new_v, sink_k=sink_k, sink_v=sink_v, max_len=max_len, ws=ws,
                out=out, bulk_ms=bulk_ms, bulk_rows=bulk_rows, n_ctx=n_ctx, num_blocks=num_blocks,
                n_queries=n_queries, multi_slots=multi_slots)


def run_step(w, S, tq, step, ev=None):
    """One step over all layers; ev maps layer -> (a0, a1, d1) events for the calls to time."""
    for l, L in enumerate(S["layers"]):
        e = None if ev is None else ev.get(l)
        if e is not None:
            e[0].record()
        if L.fused:  # the new token's append inside the decode call (a0 starts the call)
            tq.tq_paged_decode_attention_append(L.fmt.desc, S["qs"][l], S["new_k"][step, l],
                                                S["new_v"][step, l], L.pages, L.num_blocks, S["bt"],
                                                S["seq_lens"], S["max_len"], S["out"], S["ws"])
            if e is not None:
                e[2].record()
            continue
        # with a hot window the quantized token is the one leaving the window, and the new token
        # takes its row in the window (a ring: row step % W)
        if S["n_queries"] > 1:  # T new rows per sequence (the step's rows, repeated)
            T = S["n_queries"]
            tq.tq_quantize_append(L.fmt.desc, S["new_k"][step, l].repeat_interleave(T, 0),
                                  S["new_v"][step, l].repeat_interleave(T, 0), S["multi_slots"],
                                  L.pages, L.num_blocks)
        else:
            tq.tq_quantize_append(L.fmt.desc, S["new_k"][step, l], S["new_v"][step, l],
                                  S["new_slots"], L.pages, L.num_blocks)
        if L.win_k is not None:
            r = step % S["hot_window"]
            L.win_k[:, r].copy_(S["new_k"][step, l])
            L.win_v[:, r].copy_(S["new_v"][step, l])
        if e is not None:
            e[1].record()
        if S["n_queries"] > 1:
            tq.tq_paged_decode_attention_multi(L.fmt.desc, S["qs"][l], L.pages, L.num_blocks, S["bt"],
                                               S["seq_lens"], S["max_len"], S["out"], S["ws"],
                                               S["sink_k"], S["sink_v"], w.n_sink)
        elif L.win_k is None:
            tq.tq_paged_decode_attention(L.fmt.desc, S["qs"][l], L.pages, L.num_blocks, S["bt"],
                                         S["seq_lens"], S["max_len"], S["out"], S["ws"],
                                         S["sink_k"], S["sink_v"], w.n_sink)
        else:
            tq.tq_paged_decode_attention_window(L.fmt.desc, S["qs"][l], L.pages, L.num_blocks, S["bt"],
                                                S["seq_lens"], S["max_len"], S["out"], S["ws"],
                                                L.win_k, L.win_v, S["win_lens"], S["sink_k"],
                                                S["sink_v"], w.n_sink)
        if e is not None:
            e[2].record()


def algorithmic_bytes(w, lens, tq, win_lens=None, n_queries=1, flags=0):
    """Bytes the decode of one layer must move (with a hot window of win_lens[b] fp16 rows; with
    n_queries queries per sequence, that many query and output rows)."""
    B, H, D = w.num_seqs, w.num_kv_heads, w.head_dim
    win = np.zeros_like(lens) if win_lens is None else np.asarray(win_lens)
    per_layer = []
    for l in range(w.layers):
        kb, vb = w.bits(l)
        sb = tq.tq_slot_bytes_ex(D, kb, vb, flags)
        page_tok = np.maximum(lens - w.n_sink - win, 0)
        b = int(page_tok.sum()) * H * sb                                  # packed slots
        b += int(win.sum()) * H * D * 2 * 2                               # fp16 window rows
        b += int(np.sum((lens + w.block_size - 1) // w.block_size)) * 4   # block tables
        b += n_queries * B * w.num_q_heads * D * (2 + 4) + B * 4          # q, out, seq_lens
        b += B * w.n_sink * H * D * 2 * 2                                 # fp16 sinks
        per_layer.append(b)
    return per_layer


DECODE_SOURCES = ("tq_decode.hip", "tq_decode_block.hip", "tq_device.h", "tq_internal.h",
                  "tq_quant_device.h")


def decode_source_digest():
    """sha256 over the decode kernels' sources: recorded traffic is only valid for this code."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "packed_decode_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(w):
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary of
    this workload, or None when there is none or the decode sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"decode_{w.name}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                kv[parts[0]] = parts[1]
    if kv.get("source_sha256") != decode_source_digest() or "traffic_bytes_per_call" not in kv:
        return None
    return float(kv["traffic_bytes_per_call"])


def copy_probe(torch, mib):
    """A plain device-to-device copy of known size, the calibration run for the HBM counters."""
    n = mib << 20
    src = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "dispatches": 4}), flush=True)


def stream_probe(torch, tq, w, reps=10):
    """Streaming ceilings from the diagnostic kernel of include/tq_probe.h, no compute: the page
    tensor of workload w read in a random block order in units of the block decode kernel's split
    size, the same tensor in place order, and a 4:1 read:write stream the size of the bulk
    quantize-append's traffic.  One JSON line."""
    from packed_decode_attention_amd import workloads as wl
    lens = wl.seq_lens(w)
    kb, vb = w.bits(w.layers // 2)  # the format of most layers
    slot = tq.tq_slot_bytes(w.head_dim, kb, vb)
    block_bytes = w.block_size * w.num_kv_heads * slot
    usable = (block_bytes // 1024) * 1024
    n_blocks = int(sum((int(L) + w.block_size - 1) // w.block_size for L in lens))
    chunk = -(-int(lens.sum()) // 256)
    chunk = -(-chunk // 16) * 16
    per_unit = max(1, chunk // w.block_size)
    gen = torch.Generator().manual_seed(7)
    order = torch.randperm(n_blocks, generator=gen).to(torch.int32).cuda()
    src = torch.full((n_blocks * usable,), 0x11, dtype=torch.uint8, device="cuda")

    def timeit(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return min(ts), float(np.mean(ts))

    out = {"probe": "stream", "workload": w.name, "block_bytes_read": usable, "blocks": n_blocks,
           "blocks_per_unit": per_unit}
    for name, od in (("random_block_order", order), ("in_place_order", None)):
        best, mean = timeit(lambda: tq.tq_probe_stream(src, n_blocks, usable, od, per_unit))
        out[name] = {"bytes": n_blocks * usable, "best_us": best, "mean_us": mean,
                     "best_GBps": n_blocks * usable / best / 1e3, "frac": n_blocks * usable / best / 1e3 / HBM_PEAK_GBS}
    del src
    # 4:1 read:write, 16 KB read blocks, about the bulk fill's bytes (fp16 K and V rows in, slots out)
    n4 = (int(lens.sum()) * w.num_kv_heads * 4 * w.head_dim) // 16384
    src4 = torch.full((n4 * 16384,), 0x22, dtype=torch.uint8, device="cuda")
    dst4 = torch.empty((n4 * 4096,), dtype=torch.uint8, device="cuda")
    best, mean = timeit(lambda: tq.tq_probe_stream(src4, n4, 16384, None, max(1, n4 // 256), dst4, 4))
    moved = n4 * (16384 + 4096)
    out["read4_write1"] = {"bytes": moved, "best_us": best, "mean_us": mean, "best_GBps": moved / best / 1e3,
                           "frac": moved / best / 1e3 / HBM_PEAK_GBS}
    print(json.dumps(out), flush=True)


CPU_MAX_TOKENS = 32769  # tokens of a sequence in the CPU sample: its first ones, up to one
                        # Llama-shaped sequence (the oracle builds 8-bit pages about 13x slower
                        # than 4-bit ones)


def cpu_sample_layer(w):
    """The first layer in the workload's main page format."""
    return next(l for l in range(w.layers) if w.bits(l) == (w.k_bits, w.v_bits))


def _oracle_sequence(w, b, before_decode=None):
    """The first CPU_MAX_TOKENS tokens of sequence b (a shorter sequence of the same layer)
    through the oracle as it stands: its pages built by the oracle's quantizer, then its decode.
    `before_decode`, if given, is called between the two.  Returns (tokens, quantize seconds, rows,
    decode start, decode end), times on the system-wide monotonic clock."""
    from oracle import attention as oatt
    from oracle import codebook as ocb
    from oracle import quantize as oq
    from packed_decode_attention_amd import workloads as wl

    lens = wl.seq_lens(w)
    l = cpu_sample_layer(w)
    kb, vb = w.bits(l)
    ck, cv = ocb.codebook(w.head_dim, kb), ocb.codebook(w.head_dim, vb)
    layer = dict(D=w.head_dim, H_kv=w.num_kv_heads, block_size=w.block_size, k_bits=kb, v_bits=vb, seed=0)
    q = wl.queries(w, l).numpy()
    sk, sv = wl.sinks(w, l)
    L = min(int(lens[b]), CPU_MAX_TOKENS)
    one = wl.scaled(w, num_seqs=1)
    bt1, nblk = wl.block_tables(one, np.array([L]))
    pages = np.zeros(nblk * w.block_size * w.num_kv_heads * oq.slot_bytes(w.head_dim, kb, vb), np.uint8)
    k = wl.kv_values(w, l, L, "k").numpy()
    v = wl.kv_values(w, l, L, "v").numpy()
    slots = wl.token_slots(bt1, 0, np.arange(L), w.block_size)
    clock = time.CLOCK_MONOTONIC
    t0 = time.clock_gettime(clock)
    oq.append_rows_fast(pages, k, v, slots, ck.boundaries32, cv.boundaries32, kb, vb, 0)
    tq_s = time.clock_gettime(clock) - t0
    if before_decode is not None:
        before_decode()
    t1 = time.clock_gettime(clock)
    oatt.decode_attention(q[b:b + 1], pages, bt1, np.array([L]), layer, ck.centroids32, cv.centroids32,
                          None if sk is None else sk.numpy()[b:b + 1],
                          None if sv is None else sv.numpy()[b:b + 1], w.n_sink)
    t2 = time.clock_gettime(clock)
    return L, tq_s, L * w.num_kv_heads, t1, t2


def _oracle_worker_init(barrier):
    """One thread per worker process: BLAS and torch's CPU pool (the seeded input generators)."""
    import threadpoolctl
    import torch
    torch.set_num_threads(1)
    globals()["_pool_limits"] = threadpoolctl.threadpool_limits(limits=1)
    globals()["_pool_barrier"] = barrier


def _oracle_worker(name, b):
    """One sequence in a worker: its pages, then a wait for every worker's pages, then its decode.
    (A worker blocked at the barrier takes no other task, so the tasks go to distinct workers.)"""
    from packed_decode_attention_amd import workloads as wl
    return _oracle_sequence(wl.WORKLOADS[name], b, before_decode=_pool_barrier.wait)


def cpu_baseline_run(w, budget_s):
    """One thread: the first sequences in turn until about `budget_s` seconds of oracle work have
    been timed."""
    tokens, t_dec, t_q, rows_q, seqs = 0, 0.0, 0.0, 0, []
    for b in range(w.num_seqs):
        L, tq_s, rows, d0, d1 = _oracle_sequence(w, b)
        t_q += tq_s
        rows_q += rows
        t_dec += d1 - d0
        tokens += L
        seqs.append(b)
        log(f"oracle, one thread: sequence {b} done ({L} tokens)")
        if t_dec + t_q > budget_s:
            break
    return tokens / t_dec, tokens, seqs, rows_q / t_q


def cpu_host_threads():
    """Logical CPUs this process may run on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_pool(w, workers):
    """All host threads: one worker process per sequence, each on one thread, up to `workers`
    sequences.  The workers build their pages, meet at a barrier, then decode side by side; the
    rate is the sequences' tokens over the span from the first decode's start to the last one's
    end."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    seqs = list(range(min(workers, w.num_seqs)))
    ctx = multiprocessing.get_context("spawn")  # fresh interpreters: nothing inherited from this one
    barrier = ctx.Barrier(len(seqs), timeout=900)
    from concurrent.futures import as_completed
    res = []
    with ProcessPoolExecutor(max_workers=len(seqs), mp_context=ctx, initializer=_oracle_worker_init,
                             initargs=(barrier,)) as ex:
        for f in as_completed([ex.submit(_oracle_worker, w.name, b) for b in seqs]):
            res.append(f.result())
            log(f"oracle, {len(seqs)} processes: {len(res)} of {len(seqs)} sequences done")
    tokens = sum(r[0] for r in res)
    span = max(r[4] for r in res) - min(r[3] for r in res)
    rows = sum(r[2] for r in res)
    q_rate = rows / max(r[1] for r in res)  # the page builds overlap too: rows over the longest
    return tokens / span, tokens, seqs, len(seqs), q_rate


def cpu_baseline(w, budget_s=12.0):
    """The oracle timed on the host twice: on one thread, then with one worker process per
    sequence on every host thread (up to 16).  Run before this process touches the GPU."""
    import threadpoolctl
    import torch
    nt = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpoolctl.threadpool_limits(limits=1):
            v1, tok1, seqs1, rq1 = cpu_baseline_run(w, budget_s)
    finally:
        torch.set_num_threads(nt)
    vn, tokn, seqsn, procs, rqn = cpu_baseline_pool(w, cpu_host_threads())

    def sample(tokens, seqs, rows_rate):
        return (f"layer {cpu_sample_layer(w)} (K{w.k_bits}/V{w.v_bits}) decode of the first {CPU_MAX_TOKENS} "
                f"tokens at most of sequences {seqs} ({tokens} KV tokens, {w.num_kv_heads} kv heads, "
                f"{w.num_q_heads} q heads) with the fp64 NumPy oracle; its quantize of the same rows ran at "
                f"{rows_rate:.0f} rows/s")
    return {"value": vn, "unit": "KV tokens/s", "cores": int(procs), "kind": "oracle",
            "sample": sample(tokn, seqsn, rqn) + f"; {procs} worker processes of one thread each, one "
                      f"sequence apiece, decoding side by side on a host with {os.cpu_count()} logical CPUs",
            "one_thread": {"value": v1, "unit": "KV tokens/s", "cores": 1,
                           "sample": sample(tok1, seqs1, rq1) + "; one thread"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (the GPU clock settles within the first few hundred "
                         "milliseconds of load)")
    ap.add_argument("--workload", default="llama3-8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work per CPU baseline run (two runs: 1 thread, all threads)")
    ap.add_argument("--hot-window", type=int, default=0, metavar="W",
                    help="keep the last W tokens of each sequence as fp16 rows (decode through "
                         "tq_paged_decode_attention_window)")
    ap.add_argument("--norm-correction", action="store_true",
                    help="store corrected norms n / ||c[idx]|| (the norm-correction page format)")
    ap.add_argument("--mean-removal", action="store_true",
                    help="centre each row and store its mean (the mean-removal page format)")
    ap.add_argument("--qjl", action="store_true",
                    help="keys carry a 1-bit residual sketch and its norm (the QJL key format; keys "
                         "of 2-4 bits)")
    ap.add_argument("--queries", type=int, default=1, metavar="T",
                    help="decode T causal queries per sequence (its last T positions) per call, "
                         "through tq_paged_decode_attention_multi")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM counter calibration)")
    ap.add_argument("--separate-append", action="store_true",
                    help="time tq_quantize_append and tq_paged_decode_attention as two calls even "
                         "where the fused call serves the format")
    ap.add_argument("--graph", action="store_true",
                    help="also replay each timed step as one captured HIP graph (the host launches "
                         "one graph per step instead of every kernel); value and ms_per_step are "
                         "then the replayed steps'")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only measure the streaming ceilings of the workload's access patterns "
                         "(the diagnostic kernel of include/tq_probe.h)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import packed_decode_attention_amd as tq
    from packed_decode_attention_amd import workloads as wl

    cpu = None
    if not (args.no_cpu_baseline or args.copy_probe or args.stream_probe):
        # before the GPU is touched: the worker processes start as fresh interpreters
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl.WORKLOADS[args.workload], args.cpu_budget)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
        return
    w = wl.WORKLOADS[args.workload]
    if args.stream_probe:
        stream_probe(torch, tq, w)
        return
    log(f"workload {describe(w)}")
    total = args.warmup + args.steps
    t0 = time.time()
    if args.queries > 1 and args.hot_window:
        sys.exit("--queries and --hot-window do not combine (the multi-query call has no window)")
    if args.qjl and max(max(w.bits(l)[0] for l in range(w.layers)), w.k_bits) > 4:
        sys.exit(f"--qjl needs keys of 2-4 bits; workload {w.name} has wider keys")
    S = setup(w, torch, tq, wl, total, args.hot_window, args.norm_correction, args.queries,
              args.mean_removal, args.qjl, not args.separate_append)
    fused = [L.fused for L in S["layers"]]
    log(f"setup done in {time.time() - t0:.1f}s (bulk fill of {w.layers} layers)")

    for s in range(args.warmup):
        run_step(w, S, tq, s)
    torch.cuda.synchronize()
    log("warmup done")

    # HIP events around the calls of one layer in eight per timed step (step s times layers
    # s mod 8, s mod 8 + 8, ...): an event between two launches costs the stream a few
    # microseconds, which events around every call would add to the step time
    sampled = []  # (layer, (a0, a1, d1))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        ev = {l: tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
              for l in range(s % 8, w.layers, 8)}
        sampled += list(ev.items())
        run_step(w, S, tq, args.warmup + s, ev)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    fused_l = [S["layers"][l].fused for l, _ in sampled]
    dec_ms = np.array([(e[0] if f else e[1]).elapsed_time(e[2]) for f, (_, e) in zip(fused_l, sampled)])
    app_ms = np.array([0.0 if f else e[0].elapsed_time(e[1]) for f, (_, e) in zip(fused_l, sampled)])
    n = len(sampled)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; "
        f"{'append + decode' if all(fused) else 'decode'} {dec_ms.mean() * 1e3:.1f} us/layer "
        f"(p10 {np.percentile(dec_ms, 10) * 1e3:.1f}, p90 {np.percentile(dec_ms, 90) * 1e3:.1f}); "
        + ("append fused into the decode call" if all(fused) else f"append {app_ms.mean() * 1e3:.1f} us/layer"))

    eager_ms_per_step = ms_per_step
    if args.graph:
        # the same steps (same inputs, same slots) captured one graph each, replayed once untimed,
        # then timed; every kernel of the eager step runs in the replay
        graphs = []
        for s in range(args.steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(w, S, tq, args.warmup + s)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        start.record()
        for g in graphs:
            g.replay()
        stop.record()
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(stop) / args.steps
        log(f"graph replay of the {args.steps} steps: {ms_per_step:.3f} ms/step "
            f"(eager {eager_ms_per_step:.3f})")

    lens = S["lens"]
    kv_tokens_step = int(lens.sum()) * w.layers
    value = kv_tokens_step / (ms_per_step / 1e3)
    fmt_flags = (tq.TQ_FLAG_NORM_CORRECTION if args.norm_correction else 0) | \
                (tq.TQ_FLAG_MEAN_REMOVAL if args.mean_removal else 0) | \
                (tq.TQ_FLAG_QJL if args.qjl else 0)
    per_layer_bytes = algorithmic_bytes(w, lens, tq, S["win_lens_np"] if args.hot_window else None,
                                        args.queries, fmt_flags)
    # a fused call also reads the new rows and writes their slots
    app_bytes = [w.num_seqs * w.num_kv_heads * (4 * w.head_dim + tq.tq_slot_bytes_ex(w.head_dim, *w.bits(l), fmt_flags))
                 if fused[l] else 0 for l in range(w.layers)]
    layer_ids = [l for l, _ in sampled]
    dec_bytes = np.array([per_layer_bytes[i] + app_bytes[i] for i in layer_ids], np.float64)
    achieved = float(dec_bytes.sum() / (dec_ms.sum() / 1e3) / 1e9)
    bulk_ms = float(np.mean(S["bulk_ms"])) if S["bulk_ms"] else float("nan")
    kb, vb = w.bits(1 % w.layers)
    bulk_bytes = (S["n_ctx"] * w.num_kv_heads * (4 * w.head_dim + tq.tq_slot_bytes_ex(w.head_dim, kb, vb, fmt_flags))
                  + S["n_ctx"] * 8)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 hi+lo MFMA operands, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": describe(w) + (f", fp16 hot window of {args.hot_window} tokens"
                                             if args.hot_window else "")
                               + (", norm-correction format" if args.norm_correction else "")
                               + (", mean-removal format" if args.mean_removal else "")
                               + (", QJL key format" if args.qjl else "")
                               + (f", {args.queries} causal queries per sequence" if args.queries > 1 else ""),
                   "kv_tokens_per_layer": int(lens.sum()),
                   "layers": w.layers, "step": "per layer: quantize-append 1 token/seq + paged decode attention"
                   + (", each step replayed as one captured HIP graph" if args.graph else "")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (None if (args.hot_window or args.queries > 1 or args.mean_removal
                                          or args.qjl) else recorded_traffic(w)),
                     "kernel": ("append + decode call (tq_paged_decode_attention_append): " if all(fused)
                                else "decode call: ") + " + ".join(tq.decode_kernel_names(
                         w.head_dim, w.k_bits, w.v_bits, args.qjl, w.num_kv_heads, w.group, fmt_flags)),
                     "bytes_per_launch": float(np.mean(dec_bytes)),
                     "avg_launch_us": float(dec_ms.mean() * 1e3)},
        "append": {"fused_into_decode": bool(all(fused)),
                   "step_us_per_layer": None if all(fused) else float(app_ms.mean() * 1e3),
                   "bulk_fill_us_per_layer": bulk_ms * 1e3,
                   "bulk_fill_GBps": bulk_bytes / (bulk_ms / 1e3) / 1e9,
                   "bulk_fill_frac": bulk_bytes / (bulk_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                   "bulk_rows": S["bulk_rows"]},
    }
    if args.graph:
        result["eager_ms_per_step"] = eager_ms_per_step
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
