"""TurboQuant packed-KV hot path on AMD Instinct MI355X (gfx950).

The compute lives in the HIP library libtq.so (include/tq.h).  This package is its thin Python
binding: `_lib` mirrors the C ABI one function per entry point; `LayerFormat` builds a layer
descriptor with its device codebooks; `workloads` generates the seeded synthetic inputs.

PyTorch provides device memory and streams only.  Nothing here computes any step of the method.
"""

from __future__ import annotations

import numpy as np

from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    TqError,
    tq_build_codebook,
    TQ_APPEND_MAX_SEQS,
    TQ_MAX_QUERIES,
    tq_decode_multi_workspace_bytes,
    tq_decode_workspace_bytes,
    tq_dequantize_rows,
    tq_layer_desc,
    tq_paged_decode_attention,
    tq_paged_decode_attention_multi,
    tq_paged_decode_attention_noalloc,
    tq_paged_decode_attention_append,
    tq_paged_decode_attention_window,
    tq_probe_stream,
    tq_quantize_append,
    tq_rht_signs,
    tq_slot_bytes,
    tq_slot_bytes_ex,
    tq_status_str,
)

TQ_FLAG_NORM_CORRECTION = 1  # tq_layer_desc.flags: stored norms are n / ||c[idx]|| (include/tq.h)
TQ_FLAG_MEAN_REMOVAL = 2     # tq_layer_desc.flags: rows centred, the mean stored after the norm
TQ_FLAG_QJL = 4              # tq_layer_desc.flags: keys carry a 1-bit residual sketch and its norm

_CODEBOOKS: dict = {}


def host_codebook(D: int, bits: int, family: str = "beta"):
    """fp32 (centroids, boundaries) from tq_build_codebook, memoised per (D, bits, family)."""
    key = (D, bits, family)
    if key not in _CODEBOOKS:
        c, t, _, _, _ = tq_build_codebook(D, bits, family)
        _CODEBOOKS[key] = (c, t)
    return _CODEBOOKS[key]


class LayerFormat:
    """One layer's TQ format (head_dim, heads, bits, block size, slot stride, rotation seed)
    plus its fp32 codebooks on the device.  Keeps the device arrays alive for `desc`."""

    def __init__(self, head_dim: int, num_q_heads: int, num_kv_heads: int, k_bits: int,
                 v_bits: int, block_size: int = 16, rht_seed: int = 0, family: str = "beta",
                 slot_stride: int = 0, device="cuda", k_codebook=None, v_codebook=None,
                 norm_correction: bool = False, mean_removal: bool = False, qjl: bool = False):
        import torch
        self.head_dim, self.num_q_heads, self.num_kv_heads = head_dim, num_q_heads, num_kv_heads
        self.k_bits, self.v_bits, self.block_size = k_bits, v_bits, block_size
        self.rht_seed, self.family = rht_seed, family
        self.norm_correction, self.mean_removal, self.qjl = norm_correction, mean_removal, qjl
        self.flags = ((TQ_FLAG_NORM_CORRECTION if norm_correction else 0)
                      | (TQ_FLAG_MEAN_REMOVAL if mean_removal else 0)
                      | (TQ_FLAG_QJL if qjl else 0))
        self.slot_bytes = tq_slot_bytes_ex(head_dim, k_bits, v_bits, self.flags)
        self.slot_stride = slot_stride or self.slot_bytes
        kc, kt = k_codebook if k_codebook is not None else host_codebook(head_dim, k_bits, family)
        vc, vt = v_codebook if v_codebook is not None else host_codebook(head_dim, v_bits, family)
        as_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
        self.k_centroids, self.k_boundaries = as_dev(kc), as_dev(kt)
        if np.array_equal(np.asarray(kc, np.float32), np.asarray(vc, np.float32)) and \
                np.array_equal(np.asarray(kt, np.float32), np.asarray(vt, np.float32)):
            # one codebook for K and V: one device array, which lets decode keep one LDS table
            self.v_centroids, self.v_boundaries = self.k_centroids, self.k_boundaries
        else:
            self.v_centroids, self.v_boundaries = as_dev(vc), as_dev(vt)
        self.desc = tq_layer_desc(
            head_dim=head_dim, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
            block_size=block_size, k_bits=k_bits, v_bits=v_bits, slot_stride=slot_stride,
            flags=self.flags, rht_seed=rht_seed,
            k_centroids=self.k_centroids.data_ptr(), k_boundaries=self.k_boundaries.data_ptr(),
            v_centroids=self.v_centroids.data_ptr(), v_boundaries=self.v_boundaries.data_ptr())

    def new_pages(self, num_blocks: int, device="cuda"):
        import torch
        return torch.zeros((num_blocks, self.block_size, self.num_kv_heads, self.slot_stride),
                           dtype=torch.uint8, device=device)

    def new_workspace(self, num_seqs: int, max_seq_len: int, device="cuda", n_queries: int = 0):
        """Decode workspace for up to num_seqs sequences of at most max_seq_len tokens (with
        n_queries > 0: for tq_paged_decode_attention_multi with that many queries)."""
        import torch
        if n_queries > 0:
            n = tq_decode_multi_workspace_bytes(self.desc, num_seqs, max_seq_len, n_queries)
        else:
            n = tq_decode_workspace_bytes(self.desc, num_seqs, max_seq_len)
        return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def decode_kernel_names(head_dim: int, k_bits: int, v_bits: int, qjl: bool = False,
                        num_kv_heads: int = 0, group: int = 0, flags: int = 0):
    """Names of the kernels one tq_paged_decode_attention call launches for this format, in
    launch order (as they appear in a kernel trace)."""
    if (head_dim == 128 and num_kv_heads == 8 and flags & ~1 == 0 and not qjl and  # unpadded slots,
            ((k_bits, v_bits) == (4, 4) and 0 < group <= 4 or  # page blocks of whole 16-position runs
             (k_bits, v_bits) == (3, 2) and 0 < group <= 8)):
        return ["tq_decode_block_kernel", "tq_decode_merge_kernel"]
    mfma = ((head_dim == 128 and k_bits in (2, 3, 4, 8) and v_bits in (2, 4, 8)) or
            (head_dim == 64 and k_bits in (4, 8) and v_bits in (4, 8)))
    return ["tq_decode_mfma_kernel" if mfma else "tq_decode_split_kernel", "tq_decode_merge_kernel"]
