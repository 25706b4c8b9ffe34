"""Decode attention over packed TQ pages (oracle, fp64, dense).

Follows:
* TorbuQuant docs, "Current Status" table: diagnostic attention routes (dense, dequantized,
  direct-QK, packed-V) and a paged decode reference over TQ packed pages; "TQ4 page tensor"
  figure for slot addressing through a block table.
* turboquant-pro 1.4.2, "Fused CUDA decode": one decode step over the whole cache computed on
  the codes equals decompress-then-attend (exact to a few 1e-7 there).
* tq-kv, "3-Fix for GGUF Models" (the first four tokens stay fp16: sink tokens; the current
  token is kept lossless) and the "Quick Start" calls pre_rotate_query_with_signs /
  fused_attention_scores (scores on the codes with a rotated query).
* turboquant-pro 1.4.2, "Streaming cache" (an uncompressed hot window of recent tokens in front
  of the bit-packed older ones) and "Fused CUDA decode" (the fp16 hot window is merged with the
  packed segment by online softmax).

Plain definition used here
--------------------------
For sequence b with L_b cached tokens and query head h (kv head h_kv = h // G, G = H_q / H_kv),
with ns = min(n_sink, L_b) sinks and the last w_b = win_lens[b] positions in the hot window
(0 <= w_b <= L_b - ns):
  k_p, v_p = the fp16 sink rows for p < ns,
             the fp16 window rows for p >= L_b - w_b (held in any order: attention does not
             depend on the order of its tokens),
             else the dequantized rows n R^T c[idx] read from page[bt[b][p // bs], p % bs, h_kv, :];
  s_p = scale * q_h . k_p      (scale = 1/sqrt(D) unless given);
  o_h = sum_p softmax(s)_p v_p over p in [0, L_b);  L_b = 0 gives o_h = 0.
Everything is fp64; the query is the fp16 input.

Several queries per sequence (decode_attention_multi): the last T cached positions of sequence b
are T new tokens whose rows are already in the cache (a speculative draft being verified, or a
chunk of a prompt); query j sits at position L_b - T + j and attends positions 0 .. L_b - T + j
(causal order), which is the single-query definition above with L_b - T + j + 1 cached tokens
(none when that is <= 0).

The second route, decode_attention_rotated(), is the fused identity a kernel uses
(q . (n R^T c) = n (R q) . c and sum_p w_p n_p R^T c_p = R^T sum_p w_p n_p c_p); the tests check
the two routes against each other by brute force.
"""

from __future__ import annotations

import numpy as np

from . import qjl, quantize, rotation


def _read(pages, slots, layer):
    """(k_idx, k_n, v_idx, v_n, k_mu, v_mu, k_bits, k_gamma) of the slots; the means are None
    without mean removal, the QJL sketch bits and residual norms None without the QJL key format."""
    mean, qjl_on = layer.get("mean", False), layer.get("qjl", False)
    r = quantize.read_slots(pages, slots, layer["H_kv"], layer["D"], layer["k_bits"], layer["v_bits"],
                            layer.get("slot_stride"), mean, qjl_on)
    if not mean:
        r = r[:4] + (None, None) + r[4:]
    return r if qjl_on else r + (None, None)


def _dequantized_sequence(pages, block_table, end, n_sink, layer, k_centroids32, v_centroids32):
    """Dequantized K, V rows [end - n_sink, H_kv, D] (fp64, plain route), positions n_sink..end-1."""
    bs = layer["block_size"]
    pos = np.arange(n_sink, end, dtype=np.int64)
    slots = np.asarray(block_table, dtype=np.int64)[pos // bs] * bs + pos % bs
    k_idx, k_n, v_idx, v_n, k_mu, v_mu, k_bits, k_gamma = _read(pages, slots, layer)
    K = quantize.dequantize_plain(k_idx, k_n, k_centroids32, layer["seed"], k_mu)
    if k_bits is not None:  # QJL key format: the key's dequantized residual
        K = K + qjl.residual_estimate(k_bits, k_gamma, layer["seed"])
    V = quantize.dequantize_plain(v_idx, v_n, v_centroids32, layer["seed"], v_mu)
    return K, V


def _window_len(win_lens, b, L, ns):
    w = 0 if win_lens is None else int(win_lens[b])
    assert 0 <= w <= L - ns, "the hot window holds at most the tokens after the sinks"
    return w


def decode_attention(q16, pages, block_tables, seq_lens, layer, k_centroids32, v_centroids32,
                     sink_k16=None, sink_v16=None, n_sink=0, scale=None, seqs=None,
                     win_k16=None, win_v16=None, win_lens=None):
    """Dense decode attention, fp64.  Returns out [B, H_q, D] (rows not in `seqs` stay zero).

    layer: dict with D, H_kv, block_size, k_bits, v_bits, seed and optionally slot_stride, mean
    (the mean-removal format) and qjl (the QJL key format).
    q16: [B, H_q, D] fp16.  block_tables: [B, max_blocks] int.  seq_lens: [B] int.
    sink_k16 / sink_v16: [B, n_sink, H_kv, D] fp16 (or None when n_sink == 0).
    win_k16 / win_v16: [B, win_cap, H_kv, D] fp16 and win_lens [B]: rows 0 .. win_lens[b] - 1 are
    the hot window of sequence b (None: no window).
    """
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    B, H_q, D = q.shape
    H_kv = layer["H_kv"]
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, H_q, D), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        if L == 0:
            continue
        ns = min(n_sink, L)
        w = _window_len(win_lens, b, L, ns)
        Kq, Vq = _dequantized_sequence(pages, block_tables[b], L - w, ns, layer, k_centroids32, v_centroids32)
        Ks = np.asarray(sink_k16[b, :ns], dtype=np.float16).astype(np.float64) if ns else Kq[:0]
        Vs = np.asarray(sink_v16[b, :ns], dtype=np.float16).astype(np.float64) if ns else Vq[:0]
        Kw = np.asarray(win_k16[b, :w], dtype=np.float16).astype(np.float64) if w else Kq[:0]
        Vw = np.asarray(win_v16[b, :w], dtype=np.float16).astype(np.float64) if w else Vq[:0]
        K = np.concatenate([Ks, Kq, Kw], axis=0)
        V = np.concatenate([Vs, Vq, Vw], axis=0)
        for h in range(H_q):
            hk = h // G
            s = scale * (K[:, hk, :] @ q[b, h])
            w = np.exp(s - s.max())
            w /= w.sum()
            out[b, h] = w @ V[:, hk, :]
    return out


def decode_attention_rotated(q16, pages, block_tables, seq_lens, layer, k_centroids32, v_centroids32,
                             sink_k16=None, sink_v16=None, n_sink=0, scale=None, seqs=None,
                             win_k16=None, win_v16=None, win_lens=None):
    """Same result through the rotated domain: scores n_K (R q).c_K, values R^T sum w n_V c_V; the
    fp16 rows (sinks, hot window) are scored and summed as they are."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    B, H_q, D = q.shape
    H_kv, bs = layer["H_kv"], layer["block_size"]
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    R = rotation.rotation_matrix(layer["seed"], D)
    ck = np.asarray(k_centroids32, np.float32).astype(np.float64)
    cv = np.asarray(v_centroids32, np.float32).astype(np.float64)
    out = np.zeros((B, H_q, D), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        if L == 0:
            continue
        ns = min(n_sink, L)
        w = _window_len(win_lens, b, L, ns)
        pos = np.arange(ns, L - w, dtype=np.int64)
        slots = np.asarray(block_tables[b], dtype=np.int64)[pos // bs] * bs + pos % bs
        k_idx, k_n, v_idx, v_n, k_mu, v_mu, k_bits, k_gamma = _read(pages, slots, layer)
        for h in range(H_q):
            hk = h // G
            qr = R @ q[b, h]
            s_codes = scale * k_n[:, hk].astype(np.float64) * (ck[k_idx[:, hk, :]] @ qr)
            if k_mu is not None:  # q . (x_hat + mu 1) = q . x_hat + mu sum(q)
                s_codes = s_codes + scale * k_mu[:, hk].astype(np.float64) * q[b, h].sum()
            if k_bits is not None:  # QJL: the residual's estimated part of q . k
                s_codes = s_codes + scale * qjl.score_term(qr, k_bits[:, hk], k_gamma[:, hk], layer["seed"])
            # the fp16 rows: sinks, then the hot window
            K16 = np.zeros((0, D))
            V16 = np.zeros((0, D))
            if ns:
                K16 = np.asarray(sink_k16[b, :ns, hk], np.float16).astype(np.float64)
                V16 = np.asarray(sink_v16[b, :ns, hk], np.float16).astype(np.float64)
            if w:
                K16 = np.concatenate([K16, np.asarray(win_k16[b, :w, hk], np.float16).astype(np.float64)])
                V16 = np.concatenate([V16, np.asarray(win_v16[b, :w, hk], np.float16).astype(np.float64)])
            s_16 = scale * (K16 @ q[b, h])
            m = max(s_codes.max() if s_codes.size else -np.inf, s_16.max() if s_16.size else -np.inf)
            w_codes = np.exp(s_codes - m)
            w_16 = np.exp(s_16 - m)
            l = w_codes.sum() + w_16.sum()
            acc_rot = (w_codes * v_n[:, hk].astype(np.float64)) @ cv[v_idx[:, hk, :]]
            o = R.T @ acc_rot + w_16 @ V16
            if v_mu is not None:  # sum_p w_p (v_hat_p + mu_p 1)
                o = o + w_codes @ v_mu[:, hk].astype(np.float64)
            out[b, h] = o / l
    return out


def decode_attention_multi(q16, pages, block_tables, seq_lens, layer, k_centroids32, v_centroids32,
                           sink_k16=None, sink_v16=None, n_sink=0, scale=None, seqs=None):
    """T queries per sequence at its last T positions, each causal.  q16: [B, T, H_q, D] fp16.
    Returns out [B, T, H_q, D] (fp64): out[:, j] is decode_attention() of query j over the first
    L_b - T + j + 1 positions."""
    q = np.asarray(q16, dtype=np.float16)
    B, T, H_q, D = q.shape
    out = np.zeros((B, T, H_q, D), dtype=np.float64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    for j in range(T):
        visible = np.maximum(lens - T + j + 1, 0)
        out[:, j] = decode_attention(q[:, j], pages, block_tables, visible, layer, k_centroids32,
                                     v_centroids32, sink_k16, sink_v16, n_sink, scale=scale, seqs=seqs)
    return out
