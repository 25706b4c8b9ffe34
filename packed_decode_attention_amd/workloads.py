"""Seeded synthetic workloads shaped like the pages' models (no method arithmetic here).

The pages report their KV results on Qwen2.5, Llama-3/3.1-8B, Mistral-7B and Gemma models and
on random Gaussian KV; no weights or datasets are available, so these generators stand in for
the KV tensors those models would produce, with the shapes, bit policies, value distributions
and block-table structure of five named workloads.

Every draw comes from a seeded torch.Generator, on the CPU for the small parity cases and on the
device for the full-size benchmark; the same arrays feed the HIP path and, copied to the host,
the CPU oracle.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    k_bits: int
    v_bits: int
    context: int                 # cached tokens before the decode step's append
    block_size: int = 16
    n_sink: int = 0
    values: str = "normal"       # normal | lognormal_channels | outliers | student_t
    tables: str = "permuted"     # identity | permuted | fragmented
    ragged: tuple | None = None  # (lo, hi) context lengths, uniform, per sequence
    protected: dict = field(default_factory=dict)  # layer -> (k_bits, v_bits)
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def bits(self, layer: int):
        return self.protected.get(layer, (self.k_bits, self.v_bits))


WORKLOADS = {
    # 1 layer, 1 KV head, D=128, 256 cached tokens, K4/V4, block 16, one query.
    "tiny": Workload("tiny", 1, 1, 1, 1, 128, 4, 4, 255, values="normal", tables="identity", seed=1),
    # Qwen2.5-0.5B-shaped: 24 layers, 14/2 heads, D=64, q8k-q8v, context 4096, batch 8.
    "qwen2.5-0.5b": Workload("qwen2.5-0.5b", 24, 8, 14, 2, 64, 8, 8, 4096,
                             values="lognormal_channels", seed=2),
    # Llama-3-8B-shaped: 32 layers, 32/8 heads, D=128, K4/V4, context 32768, batch 16.
    "llama3-8b": Workload("llama3-8b", 32, 16, 32, 8, 128, 4, 4, 32768, values="outliers", seed=3),
    # Mistral-7B-shaped q8k-int4v: K8/V4, first and last 2 layers K8/V8, 4 fp16 sinks, 131072.
    "mistral-7b": Workload("mistral-7b", 32, 4, 32, 8, 128, 8, 4, 131072, n_sink=4,
                           values="student_t",
                           protected={0: (8, 8), 1: (8, 8), 30: (8, 8), 31: (8, 8)}, seed=4),
    # Ragged serving batch: 256 sequences, lengths U[1024, 16384], 64/8 heads, K3/V2.
    "ragged": Workload("ragged", 32, 256, 64, 8, 128, 3, 2, 0, values="normal", tables="fragmented",
                       ragged=(1024, 16384), seed=5),
}


def generator(seed: int, device="cpu"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def seq_lens(w: Workload, append: bool = True) -> np.ndarray:
    """Cached tokens per sequence after the decode step's one-token append (sinks included)."""
    if w.ragged is None:
        lens = np.full(w.num_seqs, w.context, np.int64)
    else:
        rng = np.random.default_rng(w.seed * 7919 + 1)
        lens = rng.integers(w.ragged[0], w.ragged[1] + 1, size=w.num_seqs)
    return (lens + (1 if append else 0)).astype(np.int32)


def block_tables(w: Workload, lens: np.ndarray, slack_tokens: int = 0):
    """(block_tables int32 [B, max_blocks], num_blocks) for sequences of the given lengths.

    identity:   sequence b owns blocks b*nb .. b*nb + nb - 1 in order;
    permuted:   a random permutation of all B*nb blocks, dealt out in order;
    fragmented: a pool 1.25x the blocks needed, ids drawn without replacement across sequences.
    Unused table entries are -1.
    """
    bs = w.block_size
    need = (np.asarray(lens, np.int64) + slack_tokens + bs - 1) // bs
    max_blocks = int(need.max())
    total = int(need.sum())
    rng = np.random.default_rng(w.seed * 104729 + 3)
    if w.tables == "identity":
        ids = np.arange(total)
        num_blocks = total
    elif w.tables == "permuted":
        ids = rng.permutation(total)
        num_blocks = total
    else:
        num_blocks = int(np.ceil(total * 1.25))
        ids = rng.permutation(num_blocks)[:total]
    bt = np.full((len(lens), max_blocks), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        bt[b, :n] = ids[o:o + n]
        o += n
    return bt, num_blocks


def token_slots(bt: np.ndarray, b: int, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Slot ids of the given positions of sequence b (page addressing, no arithmetic of the method)."""
    positions = np.asarray(positions, np.int64)
    return bt[b, positions // block_size].astype(np.int64) * block_size + positions % block_size


def kv_values(w: Workload, layer: int, n_tok: int, which: str, device="cpu", gen=None):
    """fp16 K or V rows [n_tok, H_kv, D] with the workload's value distribution.

    normal:             N(0, 1)
    lognormal_channels: N(0, 1) * sigma[h, d], sigma = exp(0.5 z) drawn per (layer, kv head,
                        channel), separately for K and V
    outliers:           N(0, 1) with 4 channels per (layer, kv head) scaled by 20 (channels
                        drawn per layer, head and K/V)
    student_t:          Student-t with 4 degrees of freedom (z / sqrt(chi2_4 / 4))
    """
    import torch
    H, D = w.num_kv_heads, w.head_dim
    tag = 0 if which == "k" else 1
    if gen is None:
        gen = generator(w.seed * 1000003 + layer * 31 + tag, device)
    shape = (n_tok, H, D)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if w.values == "lognormal_channels" or w.values == "outliers":
        pg = generator(w.seed * 7777 + layer * 2 + tag, "cpu")
        if w.values == "lognormal_channels":
            sigma = torch.exp(0.5 * torch.randn((H, D), generator=pg))
            x = x * sigma.to(device)
        else:
            scale = torch.ones((H, D))
            for h in range(H):
                ch = torch.randperm(D, generator=pg)[:4]
                scale[h, ch] = 20.0
            x = x * scale.to(device)
    elif w.values == "student_t":
        chi2 = torch.zeros(shape, device=device)
        for _ in range(4):
            chi2 += torch.randn(shape, generator=gen, device=device) ** 2
        x = x / torch.sqrt(chi2 / 4.0)
    return x.to(torch.float16)


def queries(w: Workload, layer: int, step: int = 0, device="cpu"):
    """fp16 queries [B, H_q, D] ~ N(0, 1)."""
    import torch
    gen = generator(w.seed * 1000033 + layer * 131 + step, device)
    return torch.randn((w.num_seqs, w.num_q_heads, w.head_dim), generator=gen, device=device).to(torch.float16)


def sinks(w: Workload, layer: int, device="cpu"):
    """fp16 sink rows (K, V) [B, n_sink, H_kv, D], same value law as the cache."""
    import torch
    if w.n_sink == 0:
        return None, None
    n = w.num_seqs * w.n_sink
    k = kv_values(w, layer + 100000, n, "k", device).reshape(w.num_seqs, w.n_sink, w.num_kv_heads, w.head_dim)
    v = kv_values(w, layer + 100000, n, "v", device).reshape(w.num_seqs, w.n_sink, w.num_kv_heads, w.head_dim)
    return k.contiguous(), v.contiguous()


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (small parity variants of the full shapes)."""
    from dataclasses import replace
    return replace(w, **changes)
