"""Shared helpers of the GPU parity tests: build one seeded case, run the HIP path through the C ABI
and the CPU oracle on the same inputs, and compare at the three levels (packed bytes, dequantized
rows, attention output)."""

from __future__ import annotations

import numpy as np

from oracle import attention as oatt
from oracle import codebook as ocb
from oracle import qjl as oqjl
from oracle import quantize as oq

# Attention tolerance (fp32 accumulation on the GPU vs fp64 oracle): max-abs and relative L2.
ATOL = 1e-3
REL_L2 = 1e-4


def check_attention(got: np.ndarray, want: np.ndarray, seqs=None):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if seqs is not None:
        got, want = got[seqs], want[seqs]
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(got - want) / denom) if denom > 0 else float(np.linalg.norm(got))
    assert np.all(np.isfinite(got)), "non-finite attention output"
    assert max_abs <= ATOL, f"max-abs {max_abs:.3e} > {ATOL}"
    assert rel <= REL_L2, f"relative L2 {rel:.3e} > {REL_L2}"
    return max_abs, rel


def compare_pages(gpu: np.ndarray, ref: np.ndarray, slots: np.ndarray, H: int, D: int, kb: int,
                  vb: int, stride: int, k_tie: np.ndarray, v_tie: np.ndarray,
                  norm_correction=None, mean: bool = False, qjl_tie=None) -> int:
    """Packed bytes must be identical except for indices at oracle-listed ties (|u - t_j| <= 1e-6),
    where the neighbouring index is accepted.  Returns the number of accepted tie differences.

    slots: [n] slot of each token row (k_tie/v_tie are [n, H, D]); negative slots are skipped.
    norm_correction: None for the plain format, else ((k_norms, v_norms) [n, H] fp32 plain norms,
    (k_centroids, v_centroids)); a row whose indices differ at a tie must then store the corrected
    norm of its own indices.
    qjl_tie: None for keys without the residual sketch, else the oracle's sketch tie masks (bits
    [n, H, D], gamma [n, H]): on rows whose key codes match, sketch bits may differ only at sketch
    ties and the residual norm gamma only at a gamma tie, by one fp32 step; rows whose key codes
    moved at a code tie have a different residual and are not compared there.
    """
    keep = slots >= 0
    slots, k_tie, v_tie = slots[keep], k_tie[keep], v_tie[keep]
    qjl = qjl_tie is not None
    if qjl:
        qjl_tie, gamma_tie = qjl_tie[0][keep], qjl_tie[1][keep]
    if norm_correction is not None:
        (kn, vn), cents = norm_correction
        plain = (np.asarray(kn)[keep].reshape(-1), np.asarray(vn)[keep].reshape(-1))
    g = gpu.reshape(-1, H, stride)[slots]
    r = ref.reshape(-1, H, stride)[slots]
    if np.array_equal(g, r):
        return 0
    sb = oq.slot_bytes(D, kb, vb, mean, qjl)
    kr = oq.region_bytes(D, kb, mean)
    kq = oq.key_region_bytes(D, kb, mean, qjl)
    assert np.array_equal(g[:, :, sb:], r[:, :, sb:]), "padding bytes differ"
    ties = 0
    k_moved = None
    for side, (lo, hi, bits, tie) in enumerate(((0, kr, kb, k_tie), (kq, sb, vb, v_tie))):
        gb, rb = g[:, :, lo:hi].reshape(-1, hi - lo), r[:, :, lo:hi].reshape(-1, hi - lo)
        gi, gn = oq.unpack_regions(gb, D, bits)
        ri, rn = oq.unpack_regions(rb, D, bits)
        if mean:  # the row mean does not depend on the codes: always bit-exact
            assert np.array_equal(oq.unpack_means(gb, D, bits).view(np.uint32),
                                  oq.unpack_means(rb, D, bits).view(np.uint32)), "stored means differ"
        bad = gi != ri
        same = gn.view(np.uint32) == rn.view(np.uint32)
        if norm_correction is None:
            assert np.all(same), "stored norms differ"
        else:
            moved = bad.any(axis=1)
            assert np.all(same[~moved]), "stored norms differ"
            if moved.any():
                want = oq.corrected_norm(plain[side][moved], gi[moved], cents[side])
                assert np.array_equal(gn[moved].view(np.uint32), want.view(np.uint32)), \
                    "corrected norm of a row with a tie difference"
        t = tie.reshape(-1, D)
        assert np.all(t[bad]), f"{int(np.sum(bad & ~t))} index differences outside the tie band"
        assert np.all(np.abs(gi[bad] - ri[bad]) == 1)
        ties += int(bad.sum())
        if side == 0:
            k_moved = bad.any(axis=1)
    if qjl:
        gq, rq = g[:, :, kr:kq].reshape(-1, kq - kr), r[:, :, kr:kq].reshape(-1, kq - kr)
        gbits, ggam = oqjl.unpack(gq, D)
        rbits, rgam = oqjl.unpack(rq, D)
        ok = ~k_moved
        qt = qjl_tie.reshape(-1, D)[ok]
        flip = gbits[ok] != rbits[ok]
        assert np.all(qt[flip]), f"{int(np.sum(flip & ~qt))} sketch bits differ outside the tie band"
        gg, rg = ggam[ok], rgam[ok]
        gdiff = gg.view(np.uint32) != rg.view(np.uint32)
        gt = gamma_tie.reshape(-1)[ok]
        assert np.all(gt[gdiff]), f"{int(np.sum(gdiff & ~gt))} residual norms differ outside the tie band"
        assert np.all(np.abs(gg[gdiff].view(np.int32).astype(np.int64)
                             - rg[gdiff].view(np.int32).astype(np.int64)) == 1)
        ties += int(flip.sum()) + int(gdiff.sum())
    return ties


def oracle_codebooks(D, kb, vb, family="beta"):
    k = ocb.codebook(D, kb, family)
    v = ocb.codebook(D, vb, family)
    return (k.centroids32, k.boundaries32), (v.centroids32, v.boundaries32)


class Case:
    """One seeded decode case: per-sequence K/V for every cached position, queries, sinks,
    block tables, and the oracle's pages."""

    def __init__(self, w, layer=0, lens=None, slack=0, family="beta", slot_stride=0,
                 norm_correction=False, mean_removal=False, qjl=False):
        import torch
        from packed_decode_attention_amd import workloads as wl
        self.w = w
        kb, vb = w.bits(layer)
        self.kb, self.vb = kb, vb
        self.D, self.H, self.Hq = w.head_dim, w.num_kv_heads, w.num_q_heads
        self.lens = np.asarray(wl.seq_lens(w) if lens is None else lens, np.int32)
        self.bt, self.num_blocks = wl.block_tables(w, np.maximum(self.lens, 1), slack)
        self.family = family
        self.mean = mean_removal
        self.qjl = qjl
        self.slot_stride = slot_stride or oq.slot_bytes(self.D, kb, vb, mean_removal, qjl)
        n_tok = int(self.lens.sum())
        self.k = wl.kv_values(w, layer, n_tok, "k")
        self.v = wl.kv_values(w, layer, n_tok, "v")
        slots = [wl.token_slots(self.bt, b, np.arange(L), w.block_size) for b, L in enumerate(self.lens)]
        self.slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
        self.q = wl.queries(w, layer)
        self.sink_k, self.sink_v = wl.sinks(w, layer)
        (kc, kt), (vc, vt) = oracle_codebooks(self.D, kb, vb, family)
        self.kcb, self.vcb = (kc, kt), (vc, vt)
        self.layer_dict = dict(D=self.D, H_kv=self.H, block_size=w.block_size, k_bits=kb, v_bits=vb,
                               seed=0, slot_stride=self.slot_stride, mean=mean_removal, qjl=qjl)
        self.norm_correction = norm_correction
        self.pages_ref = np.zeros(self.num_blocks * w.block_size * self.H * self.slot_stride, np.uint8)
        ties = oq.append_rows_fast(
            self.pages_ref, self.k.numpy(), self.v.numpy(), self.slots, kt, vt, kb, vb, 0,
            self.slot_stride, k_centroids32=kc if norm_correction else None,
            v_centroids32=vc if norm_correction else None, mean=mean_removal,
            qjl_centroids32=kc if qjl else None)
        self.k_tie, self.v_tie = ties[0], ties[1]
        self.q_tie = ties[2] if qjl else None
        self._torch = torch

    # ---- HIP path -------------------------------------------------------------------------
    def fmt(self):
        from packed_decode_attention_amd import LayerFormat
        return LayerFormat(self.D, self.Hq, self.H, self.kb, self.vb, self.w.block_size, 0,
                           self.family, slot_stride=self.slot_stride if self.slot_stride !=
                           oq.slot_bytes(self.D, self.kb, self.vb, self.mean, self.qjl) else 0,
                           k_codebook=self.kcb, v_codebook=self.vcb,
                           norm_correction=self.norm_correction, mean_removal=self.mean, qjl=self.qjl)

    def nc_args(self):
        """compare_pages' norm_correction argument: the oracle's plain norms and the centroids."""
        if not self.norm_correction:
            return None
        def plain(x):  # the norm before the correction: of the row, or of the centred row
            return oq.centered_norm(x, oq.row_mean(x)) if self.mean else oq.norm_fp32(x)
        return (plain(self.k.numpy()), plain(self.v.numpy())), (self.kcb[0], self.vcb[0])

    def gpu_quantize(self, fmt):
        import packed_decode_attention_amd as tq
        torch = self._torch
        pages = torch.full((self.num_blocks, self.w.block_size, self.H, self.slot_stride), 0x5A,
                           dtype=torch.uint8, device="cuda")
        tq.tq_quantize_append(fmt.desc, self.k.cuda(), self.v.cuda(),
                              torch.from_numpy(self.slots).cuda(), pages, self.num_blocks)
        torch.cuda.synchronize()
        return pages

    def gpu_decode(self, fmt, pages_dev, workspace=None, scale=0.0):
        import packed_decode_attention_amd as tq
        torch = self._torch
        B = len(self.lens)
        max_len = int(self.lens.max()) if B else 0
        ws = fmt.new_workspace(B, max_len) if workspace is None else workspace
        out = torch.full((B, self.Hq, self.D), float("nan"), dtype=torch.float32, device="cuda")
        sk = None if self.sink_k is None else self.sink_k.cuda()
        sv = None if self.sink_v is None else self.sink_v.cuda()
        tq.tq_paged_decode_attention(fmt.desc, self.q.cuda(), pages_dev, self.num_blocks,
                                     torch.from_numpy(self.bt).cuda(),
                                     torch.from_numpy(self.lens).cuda(), max_len, out, ws,
                                     sk, sv, self.w.n_sink, scale)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ws

    def window(self, win_lens, win_cap, seed=0):
        """fp16 hot-window rows [B, win_cap, H, D]: rows 0 .. w_b - 1 of sequence b are its last w_b
        positions' K / V rows in a shuffled order; the rows past w_b hold large values a correct
        kernel never reads."""
        torch = self._torch
        rng = np.random.default_rng(seed)
        B = len(self.lens)
        wk = torch.full((B, win_cap, self.H, self.D), 300.0, dtype=torch.float16)
        wv = torch.full((B, win_cap, self.H, self.D), -300.0, dtype=torch.float16)
        offs = np.concatenate([[0], np.cumsum(self.lens)])
        for b, w in enumerate(win_lens):
            rows = offs[b] + int(self.lens[b]) - w + rng.permutation(w)
            wk[b, :w] = self.k[torch.from_numpy(rows)]
            wv[b, :w] = self.v[torch.from_numpy(rows)]
        return wk, wv, np.asarray(win_lens, np.int32)

    def gpu_decode_window(self, fmt, pages_dev, wk, wv, wl_):
        import packed_decode_attention_amd as tq
        torch = self._torch
        B = len(self.lens)
        max_len = int(self.lens.max()) if B else 0
        ws = fmt.new_workspace(B, max_len)
        out = torch.full((B, self.Hq, self.D), float("nan"), dtype=torch.float32, device="cuda")
        sk = None if self.sink_k is None else self.sink_k.cuda()
        sv = None if self.sink_v is None else self.sink_v.cuda()
        tq.tq_paged_decode_attention_window(fmt.desc, self.q.cuda(), pages_dev, self.num_blocks,
                                            torch.from_numpy(self.bt).cuda(),
                                            torch.from_numpy(self.lens).cuda(), max_len, out, ws,
                                            wk.cuda(), wv.cuda(), torch.from_numpy(wl_).cuda(),
                                            sk, sv, self.w.n_sink)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle_decode_window(self, wk, wv, wl_, seqs=None):
        sk = None if self.sink_k is None else self.sink_k.numpy()
        sv = None if self.sink_v is None else self.sink_v.numpy()
        return oatt.decode_attention(self.q.numpy(), self.pages_ref, self.bt, self.lens, self.layer_dict,
                                     self.kcb[0], self.vcb[0], sk, sv, self.w.n_sink, seqs=seqs,
                                     win_k16=wk.numpy(), win_v16=wv.numpy(), win_lens=wl_)

    def queries_multi(self, T):
        """fp16 queries [B, T, H_q, D]: the workload's queries of steps 0 .. T - 1."""
        from packed_decode_attention_amd import workloads as wl
        return self._torch.stack([wl.queries(self.w, 0, step) for step in range(T)], dim=1)

    def gpu_decode_multi(self, fmt, pages_dev, qm):
        import packed_decode_attention_amd as tq
        torch = self._torch
        B, T = qm.shape[0], qm.shape[1]
        max_len = int(self.lens.max()) if B else 0
        ws = fmt.new_workspace(B, max_len, n_queries=T)
        out = torch.full((B, T, self.Hq, self.D), float("nan"), dtype=torch.float32, device="cuda")
        sk = None if self.sink_k is None else self.sink_k.cuda()
        sv = None if self.sink_v is None else self.sink_v.cuda()
        tq.tq_paged_decode_attention_multi(fmt.desc, qm.cuda(), pages_dev, self.num_blocks,
                                           torch.from_numpy(self.bt).cuda(),
                                           torch.from_numpy(self.lens).cuda(), max_len, out, ws,
                                           sk, sv, self.w.n_sink)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle_decode_multi(self, qm):
        sk = None if self.sink_k is None else self.sink_k.numpy()
        sv = None if self.sink_v is None else self.sink_v.numpy()
        return oatt.decode_attention_multi(qm.numpy(), self.pages_ref, self.bt, self.lens, self.layer_dict,
                                           self.kcb[0], self.vcb[0], sk, sv, self.w.n_sink)

    def ref_pages_on_gpu(self):
        torch = self._torch
        return torch.from_numpy(self.pages_ref).cuda().reshape(
            self.num_blocks, self.w.block_size, self.H, self.slot_stride)

    # ---- oracle -----------------------------------------------------------------------------
    def oracle_decode(self, seqs=None, scale=None):
        sk = None if self.sink_k is None else self.sink_k.numpy()
        sv = None if self.sink_v is None else self.sink_v.numpy()
        return oatt.decode_attention(self.q.numpy(), self.pages_ref, self.bt, self.lens, self.layer_dict,
                                     self.kcb[0], self.vcb[0], sk, sv, self.w.n_sink, scale=scale, seqs=seqs)

    def oracle_dequant(self, slots):
        """(K, V) rows: the bit-exact fp32 routes (for the QJL key format, K's includes the
        dequantized residual sketch)."""
        r = oq.read_slots(self.pages_ref, slots, self.H, self.D, self.kb, self.vb, self.slot_stride,
                          self.mean, self.qjl)
        k_mu, v_mu = (r[4], r[5]) if self.mean else (None, None)
        if self.qjl:
            k = oqjl.dequantize_key_spec(r[0], r[1], self.kcb[0], r[-2], r[-1], 0, k_mu)
        else:
            k = oq.dequantize_spec(r[0], r[1], self.kcb[0], 0, k_mu)
        return k, oq.dequantize_spec(r[2], r[3], self.vcb[0], 0, v_mu)
