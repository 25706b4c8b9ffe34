"""CPU checks of bench.py's oracle baseline: the one-thread run and the worker-process pool (fresh
interpreters that build their pages, meet at a barrier and decode side by side) on two Qwen-shaped
sequences.  No GPU is touched."""

import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from packed_decode_attention_amd import workloads as wl  # noqa: E402


def test_one_thread_run_times_whole_sequences():
    w = wl.WORKLOADS["qwen2.5-0.5b"]
    rate, tokens, seqs, q_rate = bench.cpu_baseline_run(w, 0.0)  # stops after the first sequence
    assert seqs == [0]
    assert tokens == min(int(wl.seq_lens(w)[0]), bench.CPU_MAX_TOKENS)
    assert math.isfinite(rate) and rate > 0 and math.isfinite(q_rate) and q_rate > 0


def test_worker_pool_uses_one_process_per_sequence():
    w = wl.WORKLOADS["qwen2.5-0.5b"]
    rate, tokens, seqs, procs, q_rate = bench.cpu_baseline_pool(w, 2)
    assert seqs == [0, 1] and procs == 2
    assert tokens == sum(min(int(n), bench.CPU_MAX_TOKENS) for n in wl.seq_lens(w)[:2])
    assert math.isfinite(rate) and rate > 0 and math.isfinite(q_rate) and q_rate > 0


def test_sample_layer_is_in_the_main_format():
    for w in wl.WORKLOADS.values():
        assert w.bits(bench.cpu_sample_layer(w)) == (w.k_bits, w.v_bits)
    # the Mistral-shaped workload keeps its first two layers at K8/V8
    assert bench.cpu_sample_layer(wl.WORKLOADS["mistral-7b"]) == 2
