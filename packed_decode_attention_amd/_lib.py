"""ctypes binding of libtq.so (the HIP library).  Argument marshalling only.

Every entry point of include/tq.h has a Python function of the same name here.  Tensors are
torch tensors on the current HIP device; only their data pointers and the current stream cross
the boundary.  There is no fallback: if libtq.so is missing or fails to load, import of the
functions that need it raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("TQ_LIB", os.path.join(_HERE, "libtq.so"))

TQ_OK = 0
TQ_ERR_INVALID_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_WORKSPACE = -3
TQ_ERR_HIP = -4
TQ_ERR_NO_CONVERGENCE = -5
TQ_ERR_NOALLOC_LIMIT = -6
TQ_NOALLOC_WORKSPACE_BYTES = 64 << 20
TQ_APPEND_MAX_SEQS = 512

FAMILIES = {"beta": 0, "gaussian": 1}

EXPORTS = ("tq_build_codebook", "tq_rht_signs", "tq_slot_bytes", "tq_slot_bytes_ex", "tq_quantize_append",
           "tq_decode_workspace_bytes", "tq_paged_decode_attention", "tq_paged_decode_attention_noalloc",
           "tq_paged_decode_attention_append", "tq_paged_decode_attention_window", "tq_decode_multi_workspace_bytes",
           "tq_paged_decode_attention_multi", "tq_dequantize_rows", "tq_status_str")
TQ_MAX_QUERIES = 64
PROBE_EXPORTS = ("tq_probe_stream",)  # include/tq_probe.h (diagnostics)


class TqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({_lib().tq_status_str(status).decode()})")


class tq_layer_desc(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("k_bits", ctypes.c_int32),
        ("v_bits", ctypes.c_int32),
        ("slot_stride", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("rht_seed", ctypes.c_uint64),
        ("k_centroids", ctypes.c_void_p),
        ("k_boundaries", ctypes.c_void_p),
        ("v_centroids", ctypes.c_void_p),
        ("v_boundaries", ctypes.c_void_p),
    ]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run "
                               "`python -m packed_decode_attention_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        D = ctypes.POINTER(tq_layer_desc)
        lib.tq_build_codebook.argtypes = [I32, I32, I32, P, P, P, P, P]
        lib.tq_build_codebook.restype = ctypes.c_int
        lib.tq_rht_signs.argtypes = [I32, ctypes.c_uint64, P]
        lib.tq_rht_signs.restype = ctypes.c_int
        lib.tq_slot_bytes.argtypes = [I32, I32, I32]
        lib.tq_slot_bytes.restype = I32
        lib.tq_slot_bytes_ex.argtypes = [I32, I32, I32, I32]
        lib.tq_slot_bytes_ex.restype = I32
        lib.tq_quantize_append.argtypes = [D, P, P, P, I64, P, I64, P]
        lib.tq_quantize_append.restype = ctypes.c_int
        lib.tq_decode_workspace_bytes.argtypes = [D, I32, I32]
        lib.tq_decode_workspace_bytes.restype = SZ
        lib.tq_paged_decode_attention.argtypes = [D, P, P, I64, P, I32, P, I32, I32, P, P, I32,
                                                  ctypes.c_float, P, P, SZ, P]
        lib.tq_paged_decode_attention.restype = ctypes.c_int
        lib.tq_paged_decode_attention_noalloc.argtypes = [D, P, P, I64, P, I32, P, I32, I32, P, P,
                                                          I32, ctypes.c_float, P, P]
        lib.tq_paged_decode_attention_noalloc.restype = ctypes.c_int
        lib.tq_paged_decode_attention_append.argtypes = [D, P, P, P, P, I64, P, I32, P, I32, I32,
                                                         ctypes.c_float, P, P, SZ, P]
        lib.tq_paged_decode_attention_append.restype = ctypes.c_int
        lib.tq_paged_decode_attention_window.argtypes = [D, P, P, I64, P, I32, P, I32, I32, P, P,
                                                         I32, P, P, P, I32, ctypes.c_float, P, P,
                                                         SZ, P]
        lib.tq_paged_decode_attention_window.restype = ctypes.c_int
        lib.tq_decode_multi_workspace_bytes.argtypes = [D, I32, I32, I32]
        lib.tq_decode_multi_workspace_bytes.restype = SZ
        lib.tq_paged_decode_attention_multi.argtypes = [D, P, I32, P, I64, P, I32, P, I32, I32, P,
                                                        P, I32, ctypes.c_float, P, P, SZ, P]
        lib.tq_paged_decode_attention_multi.restype = ctypes.c_int
        lib.tq_dequantize_rows.argtypes = [D, P, I64, P, I64, P, P, P]
        lib.tq_dequantize_rows.restype = ctypes.c_int
        lib.tq_status_str.argtypes = [ctypes.c_int]
        lib.tq_status_str.restype = ctypes.c_char_p
        lib.tq_probe_stream.argtypes = [P, I64, I32, P, I32, P, I32, P]
        lib.tq_probe_stream.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _check(fn: str, status: int):
    if status != TQ_OK:
        raise TqError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------------------------
# Host-only calls
# ---------------------------------------------------------------------------------------------
def tq_build_codebook(D: int, bits: int, family: str = "beta"):
    """Returns (centroids fp32, boundaries fp32, centroids fp64, boundaries fp64, mse)."""
    L = 1 << bits
    c = np.zeros(L, np.float32)
    t = np.zeros(L - 1, np.float32)
    c64 = np.zeros(L, np.float64)
    t64 = np.zeros(L - 1, np.float64)
    mse = ctypes.c_double(0.0)
    st = _lib().tq_build_codebook(D, bits, FAMILIES[family], c.ctypes.data, t.ctypes.data,
                                  c64.ctypes.data, t64.ctypes.data, ctypes.addressof(mse))
    _check("tq_build_codebook", st)
    return c, t, c64, t64, mse.value


def tq_rht_signs(D: int, seed: int) -> np.ndarray:
    out = np.zeros(D, np.int8)
    _check("tq_rht_signs", _lib().tq_rht_signs(D, seed, out.ctypes.data))
    return out


def tq_slot_bytes(D: int, k_bits: int, v_bits: int) -> int:
    r = _lib().tq_slot_bytes(D, k_bits, v_bits)
    _check("tq_slot_bytes", min(r, 0))
    return r


def tq_slot_bytes_ex(D: int, k_bits: int, v_bits: int, flags: int) -> int:
    r = _lib().tq_slot_bytes_ex(D, k_bits, v_bits, flags)
    _check("tq_slot_bytes_ex", min(r, 0))
    return r


def tq_status_str(status: int) -> str:
    return _lib().tq_status_str(status).decode()


# ---------------------------------------------------------------------------------------------
# Device calls (enqueue on the current torch stream unless a stream is given)
# ---------------------------------------------------------------------------------------------
def tq_quantize_append(desc, k, v, slot_mapping, pages, num_blocks: int, stream=None) -> None:
    st = _lib().tq_quantize_append(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping),
                                   slot_mapping.numel(), _ptr(pages), num_blocks, _stream(stream))
    _check("tq_quantize_append", st)


def tq_decode_workspace_bytes(desc, num_seqs: int, max_seq_len: int) -> int:
    return int(_lib().tq_decode_workspace_bytes(ctypes.byref(desc), num_seqs, max_seq_len))


def tq_paged_decode_attention(desc, q, pages, num_blocks: int, block_tables, seq_lens,
                              max_seq_len: int, out, workspace, sink_k=None, sink_v=None,
                              n_sink: int = 0, scale: float = 0.0, stream=None) -> None:
    num_seqs = q.shape[0]
    max_blocks = block_tables.shape[1] if block_tables is not None else 0
    st = _lib().tq_paged_decode_attention(
        ctypes.byref(desc), _ptr(q), _ptr(pages), num_blocks, _ptr(block_tables), max_blocks,
        _ptr(seq_lens), num_seqs, max_seq_len, _ptr(sink_k), _ptr(sink_v), n_sink, scale,
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_paged_decode_attention", st)


def tq_paged_decode_attention_noalloc(desc, q, pages, num_blocks: int, block_tables, seq_lens,
                                      max_seq_len: int, out, sink_k=None, sink_v=None, n_sink: int = 0,
                                      scale: float = 0.0, stream=None) -> None:
    """tq_paged_decode_attention with the library's static workspace (no workspace argument)."""
    num_seqs = q.shape[0]
    max_blocks = block_tables.shape[1] if block_tables is not None else 0
    st = _lib().tq_paged_decode_attention_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(pages), num_blocks, _ptr(block_tables), max_blocks,
        _ptr(seq_lens), num_seqs, max_seq_len, _ptr(sink_k), _ptr(sink_v), n_sink, scale,
        _ptr(out), _stream(stream))
    _check("tq_paged_decode_attention_noalloc", st)


def tq_paged_decode_attention_append(desc, q, k_new, v_new, pages, num_blocks: int, block_tables,
                                     seq_lens, max_seq_len: int, out, workspace, scale: float = 0.0,
                                     stream=None) -> None:
    """Append the new token of every sequence (k_new, v_new [num_seqs][H_kv][D] fp16) at
    position seq_lens[b] - 1, then decode: one call, one launch of the decode kernels."""
    num_seqs = q.shape[0]
    max_blocks = block_tables.shape[1] if block_tables is not None else 0
    st = _lib().tq_paged_decode_attention_append(
        ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pages), num_blocks,
        _ptr(block_tables), max_blocks, _ptr(seq_lens), num_seqs, max_seq_len, scale, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_paged_decode_attention_append", st)


def tq_paged_decode_attention_window(desc, q, pages, num_blocks: int, block_tables, seq_lens,
                                     max_seq_len: int, out, workspace, win_k, win_v, win_lens,
                                     sink_k=None, sink_v=None, n_sink: int = 0, scale: float = 0.0,
                                     stream=None) -> None:
    """Decode with an fp16 hot window: win_k / win_v [B, win_cap, H_kv, D] fp16, win_lens [B]
    int32 (rows 0 .. win_lens[b] - 1 hold the last win_lens[b] positions of sequence b)."""
    num_seqs = q.shape[0]
    max_blocks = block_tables.shape[1] if block_tables is not None else 0
    win_cap = win_k.shape[1] if win_k is not None else 0
    st = _lib().tq_paged_decode_attention_window(
        ctypes.byref(desc), _ptr(q), _ptr(pages), num_blocks, _ptr(block_tables), max_blocks,
        _ptr(seq_lens), num_seqs, max_seq_len, _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(win_k),
        _ptr(win_v), _ptr(win_lens), win_cap, scale, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_paged_decode_attention_window", st)


def tq_decode_multi_workspace_bytes(desc, num_seqs: int, max_seq_len: int, n_queries: int) -> int:
    return int(_lib().tq_decode_multi_workspace_bytes(ctypes.byref(desc), num_seqs, max_seq_len,
                                                      n_queries))


def tq_paged_decode_attention_multi(desc, q, pages, num_blocks: int, block_tables, seq_lens,
                                    max_seq_len: int, out, workspace, sink_k=None, sink_v=None,
                                    n_sink: int = 0, scale: float = 0.0, stream=None) -> None:
    """Causal decode of the last T positions of every sequence: q [B, T, H_q, D] fp16, out
    [B, T, H_q, D] fp32."""
    num_seqs, n_queries = q.shape[0], q.shape[1]
    max_blocks = block_tables.shape[1] if block_tables is not None else 0
    st = _lib().tq_paged_decode_attention_multi(
        ctypes.byref(desc), _ptr(q), n_queries, _ptr(pages), num_blocks, _ptr(block_tables),
        max_blocks, _ptr(seq_lens), num_seqs, max_seq_len, _ptr(sink_k), _ptr(sink_v), n_sink,
        scale, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("tq_paged_decode_attention_multi", st)


def tq_dequantize_rows(desc, pages, num_blocks: int, slots, k_out, v_out, stream=None) -> None:
    st = _lib().tq_dequantize_rows(ctypes.byref(desc), _ptr(pages), num_blocks, _ptr(slots),
                                   slots.numel(), _ptr(k_out), _ptr(v_out), _stream(stream))
    _check("tq_dequantize_rows", st)


def tq_probe_stream(src, n_blocks: int, block_bytes: int, order=None, blocks_per_unit: int = 1, dst=None,
                    write_div: int = 0, stream=None) -> None:
    """include/tq_probe.h: the streaming-rate diagnostic (reads n_blocks blocks of src in the given
    order; with dst, writes block_bytes / write_div bytes per block beside the reads)."""
    st = _lib().tq_probe_stream(_ptr(src), n_blocks, block_bytes, _ptr(order) if order is not None else None,
                                blocks_per_unit, _ptr(dst) if dst is not None else None, write_div,
                                _stream(stream))
    if st != TQ_OK:
        raise TqError("tq_probe_stream", st)
