// Fused paged decode attention over packed TQ pages, gfx950.
//
// Method: scores on the codes with a rotated query, online softmax, values accumulated in the
// rotated frame and rotated back once per output (tq-kv "Quick Start": pre_rotate_query_with_signs
// and fused_attention_scores; "Custom CUDA Kernel Stack": split-KV flash decode with online
// softmax, attention on compressed KV without decompression; "3-Fix for GGUF Models": sink tokens
// kept fp16; turboquant-pro 1.4.2 "Fused CUDA decode": split-K decode on the codes).  With
// R = D^(-1/2) H diag(s):  q . (n R^T c) = n (R q) . c  and  sum_p w_p n_p R^T c_p = R^T sum_p w_p n_p c_p.
//
// Two launches:
//  1. a split kernel, one workgroup (4 waves) per (sequence, kv head, split of `chunk` page
//     tokens): tq_decode_mfma_kernel (matrix cores, further below) for the formats it covers,
//     else tq_decode_split_kernel (vector ALUs), described here.  A token row is held by P lanes (C = D/P coordinates each; P = 8, or 16 for 8 query
//     heads at D = 128), so a wave covers 64/P tokens per step and the QK dot product needs a
//     log2(P)-step DPP reduction.  The G query heads that share the kv head are processed
//     together, so each code is unpacked and looked up once for G heads.  Centroids come from
//     per-workgroup LDS tables indexed by whole bytes of codes.  Page rows are prefetched
//     kPrefetch steps ahead into registers; the block-table segment of the split sits in LDS so
//     no global load waits on another.  The online softmax keeps a running maximum per (row
//     group, head) and rescales only when it grows.  Writes (m, l, acc[D]) per split.
//  2. tq_decode_merge_kernel: one workgroup per (sequence, kv head): log-sum-exp merge of the
//     splits and the fp16 sinks, R^T by Walsh-Hadamard butterflies in LDS, division by the sum.
//
// Workgroups of the same (sequence, split) for different kv heads read adjacent bytes of the same
// page rows; the grid is laid out so that they land on the same XCD (round-robin dispatch puts
// workgroup i on XCD i % 8) and share its L2.

#include <climits>
#include <mutex>

#include "../../include/tq.h"
#include "tq_device.h"
#include "tq_quant_device.h"

namespace {
using namespace tqd;

constexpr int kNW = 4;          // waves per split workgroup
constexpr float kSent = -1.0e30f;  // finite stand-in for minus infinity in the running maxima
constexpr int kPrefetch = 4;    // page-row steps kept in flight per wave
constexpr int kMaxBtLds = 1024; // block-table entries staged in LDS per split

// Lanes per token row: 8, or 16 when 8 query heads share a kv head at D = 128, so that the
// per-lane query and accumulator registers (2 * G * C) still fit.
template <int D, int GMAX>
constexpr int lanes_per_row() { return (D == 128 && GMAX == 8) ? 16 : 8; }

struct DecodeArgs {
  TqLayer L;
  float rsqrt_d, qscale, sink_scale;
  const uint16_t* q;
  const uint8_t* pages;
  const int32_t* bt;
  int max_blocks;
  const int32_t* seq_lens;
  int chunk, max_split, n_units, bs_shift;
  int part_stride;   // partials per (sequence, kv head): max_split packed splits, then row chunks
  int row_chunks;    // fp16-row chunks launched per (sequence, kv head)
  int rows_blocks;   // workgroups of fp16-row chunks at the front of the split grid
  const uint16_t* sink_k;
  const uint16_t* sink_v;
  int n_sink;
  const uint16_t* win_k;     // hot window rows [B][win_cap][Hkv][D] fp16 (NULL: no window)
  const uint16_t* win_v;
  const int32_t* win_lens;   // [B]: valid window rows, the last positions of the sequence
  int win_cap;
  float* out;
  float* partials;   // [B][Hkv][part_stride][G][D + 2]: (m, l, acc[D]), log2 domain, rotated frame
  const int32_t* nsplit_of;  // packed partials per sequence as the block kernel wrote them, or NULL
  int merge_pre;             // packed partials expected per sequence (the merge's first batch)
  // Several queries per sequence: the kernels' G heads of a kv head are G_real query heads for
  // each of this launch's queries q0 .. q0 + G / G_real - 1 out of nq (one query: nq = 1, q0 = 0,
  // g_real = G).
  int nq, q0, g_real;
  // Fused append (k_new NULL: none): the new token of each sequence, K and V rows [B][Hkv][D]
  // fp16, quantized into the page slot of position seq_len - 1 by the last split's workgroup.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* pages_w;  // the pages, written
};

// Row (in units of D) of q and out for head v of kv head h: query q0 + v / g_real, query head
// h * g_real + v % g_real.
__device__ __forceinline__ int64_t q_row(const DecodeArgs& a, int b, int h, int v) {
  const int jq = v / a.g_real;
  return ((int64_t)b * a.nq + a.q0 + jq) * a.L.Hq + (int64_t)h * a.g_real + (v - jq * a.g_real);
}

// Positions below this are visible to head v: query j of nq sits at position seq_len - nq + j
// and attends causally (one query: seq_len).
__device__ __forceinline__ int q_limit(const DecodeArgs& a, int seq_len, int v) {
  return seq_len - a.nq + a.q0 + v / a.g_real + 1;
}

// Splits cover absolute positions [split * chunk, (split + 1) * chunk) of a sequence, up to the
// packed end; positions below n_sink are read from the sink arrays instead and are masked out of
// the splits, positions from the packed end on come from the hot window.
__device__ __forceinline__ int num_splits(int seq_len, int chunk) {
  return seq_len > 0 ? (seq_len + chunk - 1) / chunk : 1;
}

// Hot-window rows of sequence b (clamped to [0, min(win_cap, seq_len - ns)]).
__device__ __forceinline__ int window_len(const DecodeArgs& a, int b, int seq_len, int ns) {
  if (a.win_lens == nullptr) return 0;
  return max(0, min(a.win_lens[b], min(a.win_cap, seq_len - ns)));
}

// fp16 rows (sinks, then hot-window rows) of a sequence, kRowChunk at a time.
constexpr int kRowChunk = 128;

__device__ __forceinline__ int fp16_rows(const DecodeArgs& a, int b, int seq_len) {
  const int ns = min(a.n_sink, seq_len);
  return ns + window_len(a, b, seq_len, ns);
}

// Element offset of fp16 row i of (sequence b, kv head h): sink i, or window row i - ns.
template <int D>
__device__ __forceinline__ const uint16_t* fp16_row(const DecodeArgs& a, bool value, int b, int h,
                                                    int ns, int i) {
  if (i < ns) return (value ? a.sink_v : a.sink_k) + (((int64_t)b * a.n_sink + i) * a.L.Hkv + h) * D;
  return (value ? a.win_v : a.win_k) + (((int64_t)b * a.win_cap + (i - ns)) * a.L.Hkv + h) * D;
}

// One workgroup per (sequence, kv head, chunk of kRowChunk fp16 rows): a split partial of the same
// form as the packed splits' (maximum, sum, accumulator), the value sum u rotated into the frame
// of the packed accumulators once: R u = D^(-1/2) H (s * u) (R is linear, so the merge's R^T
// returns u).  LPH lanes of one DPP row hold a row, 8 coordinates each; every K and V row of the
// chunk is loaded at the start.  These workgroups lead the split kernels' grids (see fp16_chunk),
// so they run alongside the packed splits.
// LDS floats fp16_chunk needs: scores [GMAX][kRowChunk], maxima [GMAX], wave sums [kNW][GMAX][D + 1].
template <int D, int GMAX>
constexpr int fp16_chunk_lds() { return GMAX * kRowChunk + GMAX + kNW * GMAX * (D + 1); }

template <int D, int GMAX>
__device__ __forceinline__ void fp16_chunk(const DecodeArgs& a, int blk, float* lds) {
  const TqLayer& L = a.L;
  const int G = L.G;
  const int rc = blk % a.row_chunks;
  const int bh = blk / a.row_chunks;
  const int h = bh % L.Hkv, b = bh / L.Hkv;
  const int seq_len = a.seq_lens[b];
  const int ns = min(a.n_sink, seq_len);
  const int r0 = rc * kRowChunk;
  const int nr = min(fp16_rows(a, b, seq_len) - r0, kRowChunk);
  if (nr <= 0) return;  // the merge reads the chunks below ceil(rows / kRowChunk) only
  constexpr int LPH = D / 8;      // lanes per row
  constexpr int RPW = 64 / LPH;   // rows per wave step
  constexpr int NP = kWG / LPH;   // value-sum parts
  constexpr int UK = kRowChunk / (kNW * RPW);  // key rows per lane group
  constexpr int UV = kRowChunk / NP;           // value rows per part
  float(*s_s)[kRowChunk] = reinterpret_cast<float(*)[kRowChunk]>(lds);
  float* s_m = lds + GMAX * kRowChunk;
  float(*s_red)[GMAX][D + 1] = reinterpret_cast<float(*)[GMAX][D + 1]>(lds + GMAX * kRowChunk + GMAX);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane % LPH, slot = lane / LPH;
  const int part = tid / LPH;

  uint4 kraw[UK], vraw[UV];  // all rows in flight together
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    const int r = (u * kNW + wave) * RPW + slot;
    if (r < nr) kraw[u] = *reinterpret_cast<const uint4*>(fp16_row<D>(a, false, b, h, ns, r0 + r) + 8 * j);
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int r = part + u * NP;
    if (r < nr) vraw[u] = *reinterpret_cast<const uint4*>(fp16_row<D>(a, true, b, h, ns, r0 + r) + 8 * j);
  }
  auto unpack = [](const uint4& w, float (&x)[8]) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = half_bits_to_float(d[i] & 0xffffu);
      x[2 * i + 1] = half_bits_to_float(d[i] >> 16);
    }
  };
  {  // scores, log2 domain
    float qv[GMAX][8];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g < G) load8_f16(a.q + q_row(a, b, h, g) * D + 8 * j, qv[g]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[g][e] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int r = (u * kNW + wave) * RPW + slot;
      if (r < nr) {
        float kx[8];
        unpack(kraw[u], kx);
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
          float d = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(qv[g][e], kx[e], d);
          d = group_sum<LPH>(d);
          // several queries: a sink past a query's position is masked (no window then)
          if (g < G && j == 0) s_s[g][r] = r0 + r < q_limit(a, seq_len, g) ? d * a.sink_scale : kSent;
        }
      }
    }
  }
  __syncthreads();
  if (tid < 32 * GMAX) {  // maximum per head, 32 lanes each
    const int g = tid >> 5;
    float m = kSent;
    if (g < G)
      for (int r = tid & 31; r < nr; r += 32) m = fmaxf(m, s_s[g][r]);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
    if ((tid & 31) == 0) s_m[g] = m;
  }
  __syncthreads();

  // value sums: thread (part, j) takes rows part, part + NP, ... and coordinates 8 j .. 8 j + 7 of
  // every head
  float o[GMAX][8], ls[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    ls[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < UV; ++u) {
    const int r = part + u * NP;
    if (r < nr) {
      float v[8];
      unpack(vraw[u], v);
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g < G) {
          const float w = __builtin_amdgcn_exp2f(s_s[g][r] - s_m[g]);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[g][e] = fmaf(w, v[e], o[g][e]);
          ls[g] += w;
        }
      }
    }
  }
  // parts of a wave by lane exchanges, then the waves through LDS
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
#pragma unroll
      for (int m = LPH; m < 64; m <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] += __shfl_xor(o[g][e], m);
        ls[g] += __shfl_xor(ls[g], m);
      }
      if (lane < LPH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_red[wave][g][8 * j + e] = o[g][e];
        if (j == 0) s_red[wave][g][D] = ls[g];
      }
    }
  }
  __syncthreads();
  if (tid < LPH * G) {  // R u for head g, written as the chunk's partial
    const int g = tid / LPH;
    float x[8];
    float l = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    for (int w = 0; w < kNW; ++w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += s_red[w][g][8 * j + e];
      l += s_red[w][g][D];
    }
    const uint32_t sb = sign_byte(L.signs, j);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((sb >> e) & 1u) x[e] = -x[e];
    wht_row8_dpp<LPH>(x, j);
    float* part_out = a.partials + ((int64_t)bh * a.part_stride + a.max_split + rc) * G * (D + 2) +
                      (int64_t)g * (D + 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) part_out[2 + 8 * j + e] = x[e] * a.rsqrt_d;
    if (j == 0) {
      part_out[0] = s_m[g];
      part_out[1] = l;
    }
  }
}


// Raw page data of one step for one lane.
template <int NBK, int NBV>
struct Step {
  LaneCodes<NBK> k;
  LaneCodes<NBV> v;
  float kn, vn;
  float km, vm;  // row means (mean-removal format; else 0)
  uint32_t zb;   // QJL key format: the lane's sketch bits (C of them)
  float kg;      // QJL key format: the key residual's norm gamma
  int pos;       // position, or INT_MAX past the split's end
};

// QJL key format: a key's score gains gamma * sqrt(pi/2) / D * (S R q) . (2 b - 1) (the QJL
// estimator of the residual's inner product; tq-kv, "How It Works", step [5]).
constexpr float kQjlKappa = 1.2533141373155003f;  // sqrt(pi / 2)

template <int D, int KB, int VB, int GMAX, bool QJL = false>
__global__ __launch_bounds__(kWG, 2) void tq_decode_split_kernel(DecodeArgs a) {
  constexpr int P = lanes_per_row<D, GMAX>();
  constexpr int C = D / P;
  constexpr int TPW = 64 / P;           // tokens per wave per step
  constexpr int TPI = TPW * kNW;        // tokens per workgroup per step
  constexpr int NBK = C * KB / 8;       // code bytes per lane
  constexpr int NBV = C * VB / 8;
  const TqLayer& L = a.L;
  const int G = L.G;

  if ((int)blockIdx.x < a.rows_blocks) {  // fp16-row chunks lead the grid
    __shared__ float s_rows[fp16_chunk_lds<D, GMAX>()];
    fp16_chunk<D, GMAX>(a, blockIdx.x, s_rows);
    return;
  }
  // (sequence, split) units with equal index modulo 8 share an XCD across all kv heads
  const int lin = blockIdx.x - a.rows_blocks;
  const int xcd = lin & 7;
  const int rest = lin >> 3;
  const int h = rest % L.Hkv;
  const int unit = (rest / L.Hkv) * 8 + xcd;
  if (unit >= a.n_units) return;
  const int b = unit / a.max_split;
  const int split = unit - b * a.max_split;
  const int seq_len = a.seq_lens[b];
  const int ns = min(a.n_sink, seq_len);
  const int packed_end = seq_len - window_len(a, b, seq_len, ns);
  const int nsplit = num_splits(packed_end, a.chunk);
  if (split >= nsplit) return;

  __shared__ float s_klut[Lut<KB>::kFloats];
  __shared__ float s_vlut[Lut<VB>::kFloats];
  __shared__ float s_part[kNW][GMAX][D + 2];
  __shared__ int64_t s_boff[kMaxBtLds];  // byte offset of each page block's first row
  build_lut<KB>(s_klut, L.kc, threadIdx.x, kWG);
  build_lut<VB>(s_vlut, L.vc, threadIdx.x, kWG);

  const int p_begin = max(ns, split * a.chunk);
  const int p_end = min((split + 1) * a.chunk, packed_end);
  const int n_it = p_end > p_begin ? (p_end - p_begin + TPI - 1) / TPI : 0;
  auto block_of = [&](int p) { return a.bs_shift >= 0 ? (p >> a.bs_shift) : (p / L.bs); };
  const int blk0 = p_end > p_begin ? block_of(p_begin) : 0;
  const int nblk = p_end > p_begin ? block_of(p_end - 1) - blk0 + 1 : 0;  // <= kMaxBtLds (host)
  const int32_t* btg = a.bt + (int64_t)b * a.max_blocks + blk0;
  const int64_t row_bytes = (int64_t)L.Hkv * L.stride;
  for (int i = threadIdx.x; i < nblk; i += kWG) s_boff[i] = (int64_t)btg[i] * L.bs * row_bytes;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & (P - 1);
  const int sub = lane / P;

  // Rotated query qscale * H (s * q) for the G heads (qscale = scale * log2(e) / sqrt(D)):
  // scores come out in the log2 domain.
  uint32_t sbits = 0;
#pragma unroll
  for (int e = 0; e < C; e += 8) sbits |= sign_byte(L.signs, (C * j + e) / 8) << e;
  float qr[GMAX][C], qsum[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    qsum[g] = 0.0f;
    if (g < G) {
      const uint16_t* qp = a.q + q_row(a, b, h, g) * D + C * j;
#pragma unroll
      for (int e = 0; e < C; e += 8) load8_f16(qp + e, &qr[g][e]);
      if (L.mean) {  // mean-removal format: scale log2(e) sum(q), the weight of mu_K in a score
#pragma unroll
        for (int e = 0; e < C; ++e) qsum[g] += qr[g][e];
        qsum[g] = group_sum<P>(qsum[g]) * a.sink_scale;
      }
#pragma unroll
      for (int e = 0; e < C; ++e) qr[g][e] = ((sbits >> e) & 1u) ? -qr[g][e] : qr[g][e];
      wht_row<C, P>(qr[g], j);
#pragma unroll
      for (int e = 0; e < C; ++e) qr[g][e] *= a.qscale;
    } else {
#pragma unroll
      for (int e = 0; e < C; ++e) qr[g][e] = 0.0f;
    }
  }
  // QJL key format: qj = sqrt(pi/2) / D * S qr with S = H diag(sigma2), qr already R q scaled.
  // Every row group of every wave needs the same values: wave 0's first row group puts them in
  // LDS (the barrier before the main loop publishes them), where reads are broadcasts.
  __shared__ __align__(16) float s_qj[QJL ? GMAX : 1][QJL ? D : 4];
  if constexpr (QJL) {
    if (wave == 0 && sub == 0) {
      uint32_t sbits2 = 0;
#pragma unroll
      for (int e = 0; e < C; e += 8) sbits2 |= sign_byte(L.signs2, (C * j + e) / 8) << e;
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        float t[C];
#pragma unroll
        for (int e = 0; e < C; ++e) t[e] = ((sbits2 >> e) & 1u) ? -qr[g][e] : qr[g][e];
        wht_row<C, P>(t, j);
#pragma unroll
        for (int e = 0; e < C; ++e) s_qj[g][C * j + e] = t[e] * (kQjlKappa / (float)D);
      }
    }
  }

  float m[GMAX], l[GMAX], acc[GMAX][C];
  float mv[GMAX];  // mean-removal format: sums of 2^(s - m) mu_V
  int lim[GMAX];   // positions visible to each head (the end of the packed segment, or causal)
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    lim[g] = min(p_end, q_limit(a, seq_len, g));
    mv[g] = 0.0f;
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < C; ++e) acc[g][e] = 0.0f;
  }

  const int voff = L.kreg;  // V region
  const uint32_t row_bytes32 = (uint32_t)row_bytes;
  const uint8_t* head_base = a.pages + (int64_t)h * L.stride;
  __syncthreads();  // lookup tables and block-table segment ready

  // Page row of step `it` for this lane's row group; rows past the end re-read the last valid
  // row and are masked.
  auto fetch = [&](int it) {
    Step<NBK, NBV> st;
    int p = p_begin + it * TPI + wave * TPW + sub;
    st.pos = p < p_end ? p : INT_MAX;
    p = p < p_end ? p : p_end - 1;
    const int bi = block_of(p);
    const uint8_t* base = head_base + s_boff[bi - blk0] + __umul24((uint32_t)(p - bi * L.bs), row_bytes32);
    st.k = load_lane_codes<NBK>(base, j);
    st.v = load_lane_codes<NBV>(base + voff, j);
    st.kn = *reinterpret_cast<const float*>(base + L.kcode_bytes);
    st.vn = *reinterpret_cast<const float*>(base + voff + L.vcode_bytes);
    st.km = L.mean ? *reinterpret_cast<const float*>(base + L.kcode_bytes + 4) : 0.0f;
    st.vm = L.mean ? *reinterpret_cast<const float*>(base + voff + L.vcode_bytes + 4) : 0.0f;
    st.zb = 0;
    st.kg = 0.0f;
    if constexpr (QJL) {  // C sketch bits at bit C j of the sketch (C = 8 or 16)
      if constexpr (C == 16) st.zb = reinterpret_cast<const uint16_t*>(base + L.kqjl)[j];
      else st.zb = base[L.kqjl + j];
      st.kg = *reinterpret_cast<const float*>(base + L.kqjl + D / 8);
    }
    return st;
  };

  auto consume = [&](const Step<NBK, NBV>& st) {
    float kf[C];
    lookup_codes<KB, C>(st.k, s_klut, kf);
    float s[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < C; ++e) d += qr[g][e] * kf[e];
      if constexpr (QJL) {  // norm and gamma are the row's: one reduction for both parts
        float tz = 0.0f;
        int qoff = g * D + C * j;
        asm volatile("" : "+v"(qoff));  // keep the reads in the loop: hoisted, they fill registers
#pragma unroll
        for (int e = 0; e < C; e += 4) {
          const float4 w = *reinterpret_cast<const float4*>(&s_qj[0][0] + qoff + e);
          tz += ((st.zb >> e) & 1u) ? w.x : -w.x;
          tz += ((st.zb >> (e + 1)) & 1u) ? w.y : -w.y;
          tz += ((st.zb >> (e + 2)) & 1u) ? w.z : -w.z;
          tz += ((st.zb >> (e + 3)) & 1u) ? w.w : -w.w;
        }
        d = group_sum<P>(st.kn * d + st.kg * tz);
        s[g] = st.pos < lim[g] ? d + st.km * qsum[g] : -INFINITY;
      } else {
        d = group_sum<P>(d);
        s[g] = st.pos < lim[g] ? st.kn * d + st.km * qsum[g] : -INFINITY;
      }
    }
    bool grow = false;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) grow |= s[g] > m[g];
    if (grow) {
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (s[g] > m[g]) {
          const float r = __builtin_amdgcn_exp2f(m[g] - s[g]);
          l[g] *= r;
          mv[g] *= r;
#pragma unroll
          for (int e = 0; e < C; ++e) acc[g][e] *= r;
          m[g] = s[g];
        }
      }
    }
    float vf[C];
    lookup_codes<VB, C>(st.v, s_vlut, vf);
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const float pw = st.pos < lim[g] ? __builtin_amdgcn_exp2f(s[g] - m[g]) : 0.0f;
      l[g] += pw;
      mv[g] += pw * st.vm;
      const float w = pw * st.vn;
#pragma unroll
      for (int e = 0; e < C; ++e) acc[g][e] += w * vf[e];
    }
  };

  // kPF-deep register ring: slot u always holds step it0 + u (two deep for the QJL key format,
  // whose sketch bits and norms would otherwise push the registers past the file).
  constexpr int kPF = QJL ? 2 : kPrefetch;
  Step<NBK, NBV> ring[kPF];
#pragma unroll
  for (int u = 0; u < kPF; ++u)
    if (u < n_it) ring[u] = fetch(u);
  for (int it0 = 0; it0 < n_it; it0 += kPF) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      const int it = it0 + u;
      if (it < n_it) {
        const Step<NBK, NBV> cur = ring[u];
        if (it + kPF < n_it) ring[u] = fetch(it + kPF);
        consume(cur);
      }
    }
  }

  // Mean-removal format: the weighted means enter the rotated accumulator as (sum) R 1, which the
  // merge's R^T turns into (sum) 1; R 1 = D^(-1/2) H s over this lane's coordinates.
  if (L.mean) {
    float r1[C];
#pragma unroll
    for (int e = 0; e < C; ++e) r1[e] = ((sbits >> e) & 1u) ? -1.0f : 1.0f;
    wht_row<C, P>(r1, j);
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
      for (int e = 0; e < C; ++e) acc[g][e] += mv[g] * (r1[e] * a.rsqrt_d);
  }

  // Merge the row groups of the wave (lanes with equal j hold the same coordinates).
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
#pragma unroll
      for (int msk = P; msk < 64; msk <<= 1) {
        const float mo = __shfl_xor(m[g], msk);
        const float lo = __shfl_xor(l[g], msk);
        const float M = fmaxf(m[g], mo);
        const float r = (m[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m[g] - M);
        const float ro = (mo == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mo - M);
        l[g] = l[g] * r + lo * ro;
#pragma unroll
        for (int e = 0; e < C; ++e) {
          const float o = __shfl_xor(acc[g][e], msk);
          acc[g][e] = acc[g][e] * r + o * ro;
        }
        m[g] = M;
      }
      if (sub == 0) {
#pragma unroll
        for (int e = 0; e < C; ++e) s_part[wave][g][2 + C * j + e] = acc[g][e];
        if (j == 0) {
          s_part[wave][g][0] = m[g];
          s_part[wave][g][1] = l[g];
        }
      }
    }
  }
  __syncthreads();

  // Merge the waves and publish this split's partial (m, l, acc[D]).
  const int64_t bh = (int64_t)b * L.Hkv + h;
  float* part = a.partials + (bh * a.part_stride + split) * (int64_t)G * (D + 2);
  for (int i = threadIdx.x; i < G * (D + 2); i += kWG) {
    const int g = i / (D + 2), d = i % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_part[w][g][0]);
    float r;
    if (d == 0) {
      r = M;
    } else {
      r = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float mw = s_part[w][g][0];
        const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        r += s_part[w][g][d] * f;
      }
    }
    part[i] = r;
  }
}


// =============================================================================================
// Matrix-core split kernel: D = 128 with K codes of 2, 3, 4 or 8 bits and V codes of 2, 4 or 8
// bits, and D = 64 with 4- or 8-bit K and V codes.
//
// Per wave, tiles of 32 page positions (two sub-tiles of 16).  QK^T and PV run on
// v_mfma_f32_16x16x32_f16 (A: 16 rows x 32, B: 32 x 16 columns, fp32 accumulate):
//  * Rows of both products: row m <-> query head (m >> 2) + 4 ((m >> 1) & 1), fp16 part m & 1
//    (high, low), so result rows 4q + i of lane group q hold head q (i = 0, 1) and head q + 4
//    (i = 2, 3); with G <= 4 every lane group carries one head and rows of heads >= G are zero.
//  * QK: A = rotated query (two fp16 parts per head), B = key centroids of 16 tokens.  Lane
//    group q owns coordinates (D/4) q .. (D/4) q + D/4 - 1 of every token, one contiguous run of
//    code bytes.  A code index (one byte; six bits for 3-bit codes) selects from an LDS table the
//    fp16 high and low parts of one, two or four centroids, already in MFMA operand order; the
//    query operand repeats its values in the matching pattern, so every product of the two-part
//    query with the two-part centroid is accumulated in fp32 (about 22 significant bits per
//    factor instead of 11).
//  * PV: A = softmax weights w = p * n_V (two fp16 parts per head), B = value centroids with the
//    contraction running over tokens.  Value codes of the tile go through a per-wave LDS tile so
//    that lane (n, q) can gather the codes of coordinates (D/16) n .. (D/16) n + D/16 - 1 for
//    tokens 8q .. 8q + 7; 4-bit codes of two tokens (or 2-bit codes of four) are merged into one
//    byte per coordinate, so one table read yields the operand values of several tokens.
// All fp16 operands are pre-scaled by powers of two into the normal fp16 range (queries per
// head, centroid tables by 2^8, weights by 2^15); the scales are removed in fp32.  Weights use
// their own running maximum of score + log2(n_V), so they stay in (0, 1] before scaling.
// Page rows: when page blocks hold whole runs of 16 positions (UBLK) a wave fetches its tile's 32
// slots as consecutive 16-byte chunks, one tile ahead, and copies them into its own LDS stage,
// from which the code runs, the norms and the value codes of the PV transpose are read; for other
// block sizes each lane loads its own code runs and norms and the value codes pass through a
// per-wave LDS tile.
// =============================================================================================
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kLutShift = 8;    // centroid tables hold c * 2^8
constexpr int kWShift = 15;     // weights enter the PV product as w * 2^15

// Formats the matrix-core kernel implements (everything else runs on tq_decode_split_kernel).
constexpr bool mfma_format(int D, int KB, int VB) {
  return (D == 128 && (KB == 2 || KB == 3 || KB == 4 || KB == 8) && (VB == 2 || VB == 4 || VB == 8)) ||
         (D == 64 && (KB == 4 || KB == 8) && (VB == 4 || VB == 8));
}

__device__ __forceinline__ float4_t mfma_f16(const uint4& a, const uint4& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// fp16 high and low parts of x: hi = fp16(x), lo = fp16(x - hi); hi + lo carries ~22 bits of x.
__device__ __forceinline__ void split_f16(float x, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = (_Float16)x;
  const _Float16 l = (_Float16)(x - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

// Operand tables.  Index e holds the codes of V consecutive values (value v in bits
// [BITS v, BITS (v + 1)) of e); the entry is the 8 fp16 of an MFMA operand fragment for them:
//   V = 1 (8-bit codes): uint32 {hi, lo}                                  -> [h0 l0]
//   V = 2 (3-, 4-bit):   uint2  {hi0 hi1, lo0 lo1}                        -> [h0 h1 l0 l1]
//   V = 4 (2-bit):       uint4  {hi0 hi1, hi2 hi3, lo0 lo1, lo2 lo3}      -> [h0 h1 h2 h3 l0 l1 l2 l3]
// The other operand repeats its values to match: [x0 x0 x1 x1 ..], [x0 x1 x0 x1 ..] or
// [x0 x1 x2 x3 x0 x1 x2 x3].
template <int BITS> struct OpTable;
template <> struct OpTable<8> { using E = uint32_t; static constexpr int N = 256, V = 1; };
template <> struct OpTable<4> { using E = uint2; static constexpr int N = 256, V = 2; };
template <> struct OpTable<3> { using E = uint2; static constexpr int N = 64, V = 2; };
template <> struct OpTable<2> { using E = uint4; static constexpr int N = 256, V = 4; };

// Thread tid builds entry tid (every table has at most one entry per thread of a workgroup): its
// codebook values are loaded first (load_op_values), the entry is written once they are in
// (store_op_entry), so the loads can be issued early.
template <int BITS>
__device__ __forceinline__ void load_op_values(const float* __restrict__ c, int tid,
                                               float (&x)[OpTable<BITS>::V]) {
  constexpr int V = OpTable<BITS>::V, M = (1 << BITS) - 1;
  static_assert(OpTable<BITS>::N <= kWG, "one table entry per thread");
  const int e = tid < OpTable<BITS>::N ? tid : 0;
#pragma unroll
  for (int v = 0; v < V; ++v) x[v] = c[(e >> (BITS * v)) & M];
}

template <int BITS>
__device__ __forceinline__ void store_op_entry(typename OpTable<BITS>::E* t, const float (&x)[OpTable<BITS>::V],
                                               int tid) {
  constexpr int V = OpTable<BITS>::V;
  if (tid >= OpTable<BITS>::N) return;
  uint32_t hi[V], lo[V];
#pragma unroll
  for (int v = 0; v < V; ++v) split_f16(ldexpf(x[v], kLutShift), hi[v], lo[v]);
  if constexpr (V == 1) t[tid] = hi[0] | (lo[0] << 16);
  if constexpr (V == 2) t[tid] = make_uint2(hi[0] | (hi[1] << 16), lo[0] | (lo[1] << 16));
  if constexpr (V == 4)
    t[tid] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), lo[0] | (lo[1] << 16),
                        lo[2] | (lo[3] << 16));
}

// The other operand for four fp16 values given as x01 = x0 | x1 << 16 and x23 = x2 | x3 << 16.
template <int V>
__device__ __forceinline__ uint4 repeat_operand(uint32_t x01, uint32_t x23) {
  if constexpr (V == 2) return make_uint4(x01, x01, x23, x23);
  if constexpr (V == 4) return make_uint4(x01, x23, x01, x23);
  const uint32_t l01 = x01 & 0xffffu, l23 = x23 & 0xffffu;
  return make_uint4(l01 | (l01 << 16), (x01 >> 16) | (x01 & 0xffff0000u), l23 | (l23 << 16),
                    (x23 >> 16) | (x23 & 0xffff0000u));
}

// N consecutive dwords from a 4-byte aligned address.
template <int N>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 x = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = x.x;
      w[4 * i + 1] = x.y;
      w[4 * i + 2] = x.z;
      w[4 * i + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

template <int D, int KB, int VB>
struct MfmaCfg {
  static constexpr int QC = D / 4;              // coordinates per lane group in QK
  static constexpr int NMQ = D / 16;            // QK MFMAs per 16-token sub-tile
  static constexpr int PC = D / 16;             // coordinates per lane in PV (= PV MFMAs)
  static constexpr int KW = D * KB / 128;       // dwords of K codes per lane and token
  static constexpr int VW = D * VB / 128;       // dwords of V codes per lane and token
  static constexpr int VROW = D * VB / 32 + 2;  // dwords per token row of the value tile (padded)
  static constexpr int VK = OpTable<KB>::V, VV = OpTable<VB>::V;
  // weight tile: fp16 per token, or fp16 pairs (w, w) for 8-bit values (rows of 16-byte
  // multiples so a lane reads four pairs at once); rows padded against bank conflicts
  static constexpr int WROW = VV == 1 ? 36 : 18;  // dwords per weight row
};

template <int D, int KB, int VB>
struct MfmaTile {
  uint32_t k[2][MfmaCfg<D, KB, VB>::KW];  // K codes of tokens t16, 16 + t16 (lane group's run)
  uint32_t v[2][MfmaCfg<D, KB, VB>::VW];  // V codes of the same tokens and coordinates
  float kn[2], vn[2];
  float km[2], vm[2];  // row means (mean-removal format; else 0)
  uint32_t zb[2];      // QJL key format: sketch bits of the lane group's coordinates
  float kg[2];         // QJL key format: residual norms gamma
};

// Page rows of a 32-position tile for one kv head, as fetched when page blocks hold whole runs of
// 16 positions and slots are unpadded: a slot is N16 16-byte chunks and, in the plain format, an
// 8-byte tail (mean-removal slots, MEAN, are whole chunks).  Lane l fetches chunk c = 64 i + l of
// the tile (row c / N16, chunk c % N16) into c[i] and, for l < 32, the tail of row l: consecutive
// lanes read consecutive bytes of a row, so a wave's load covers 64 / N16 whole slots instead of
// a 16-byte piece of 16 slots.  In the wave's LDS stage row r starts at r * SS, with SS / 4 = 2
// mod 4 (a mean-removal slot gets 8 bytes of padding for that).
template <int D, int KB, int VB, bool MEAN = false>
struct MfmaRaw {
  static constexpr int SB = D * KB / 8 + D * VB / 8 + (MEAN ? 16 : 8);  // slot bytes
  static constexpr int TAIL = SB % 16;
  static constexpr int N16 = (SB - TAIL) / 16;
  static constexpr int NI = (32 * N16 + 63) / 64;
  static constexpr int SS = TAIL ? SB : SB + 8;  // stage row stride
  static_assert(TAIL == 8 || TAIL == 0, "slot = whole 16-byte chunks + an 8-byte tail, or chunks only");
  static_assert((SS / 4) % 4 == 2, "stage rows 2 mod 4 dwords apart");
  uint4 c[NI];
  uint2 t;
};

template <int DPPCTRL>
__device__ __forceinline__ float dpp_max_step(float x) { return fmaxf(x, dpp<DPPCTRL>(x)); }

// Maximum over aligned groups of P = 8 or 16 lanes, result in every lane of the group.
template <int P>
__device__ __forceinline__ float lanes_max(float x) {
  x = dpp_max_step<kDppQuadXor1>(x);
  x = dpp_max_step<kDppQuadXor2>(x);
  x = dpp_max_step<kDppHalfRowMirror>(x);
  if constexpr (P == 16) x = dpp_max_step<kDppRowMirror>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) { return lanes_max<16>(x); }

// B operand of QK step st (coordinates 4 st .. 4 st + 3 of the lane's run) from its code words.
template <int KB>
__device__ __forceinline__ uint4 k_operand(const typename OpTable<KB>::E* tab, const uint32_t* kw, int st) {
  if constexpr (KB == 8) {
    const uint32_t w = kw[st];
    return make_uint4(tab[w & 0xffu], tab[(w >> 8) & 0xffu], tab[(w >> 16) & 0xffu], tab[w >> 24]);
  } else if constexpr (KB == 4) {
    const uint32_t w = kw[st >> 1] >> (16 * (st & 1));
    const uint2 e0 = tab[w & 0xffu], e1 = tab[(w >> 8) & 0xffu];
    return make_uint4(e0.x, e0.y, e1.x, e1.y);
  } else if constexpr (KB == 3) {
    const int bit = 12 * st;  // two 6-bit indices at bits [12 st, 12 st + 12) of the run
    const int wi = bit >> 5, sh = bit & 31;
    const uint32_t f = sh <= 20 ? (kw[wi] >> sh) : __builtin_amdgcn_alignbit(kw[wi + 1], kw[wi], sh);
    const uint2 e0 = tab[f & 63u], e1 = tab[(f >> 6) & 63u];
    return make_uint4(e0.x, e0.y, e1.x, e1.y);
  } else {
    return tab[(kw[st >> 2] >> (8 * (st & 3))) & 0xffu];
  }
}

// Destination of the fused append's stores from the lanes of rows other than the new token's (a
// tile's lanes all store).
__device__ __align__(16) uint8_t tq_decode_append_discard[512];  // >= the largest plain slot (264 B)

// Fused append, one wave: the new token's K and V rows of kv head h of sequence b, quantized
// exactly as tq_quantize_kernel does (the same region code and Hadamard operands; decisions by
// binary search over the fp32 boundaries, which select the codes the quantizer's bucket table
// selects) into the slot of position seq_len - 1.  The wave's 16 tile rows all hold that row;
// lanes of row 0 store to the page, the others to the discard buffer.  s_t: [2][256] LDS floats
// of this wave.  The stores are complete on return.
template <int D, int KB, int VB>
__device__ __forceinline__ void append_row(const DecodeArgs& a, int b, int h, int seq_len, int lane,
                                           float (*s_t)[256]) {
  const TqLayer& L = a.L;
  constexpr int NB = D / 32;
  constexpr int nbk = (1 << KB) - 1, nbv = (1 << VB) - 1;
  const int c = lane & 15, g = lane >> 4;
  const uint16_t* sk = a.k_new + ((int64_t)b * L.Hkv + h) * D + 8 * g;
  const uint16_t* sv = a.v_new + ((int64_t)b * L.Hkv + h) * D + 8 * g;
  uint4 xk[NB], xv[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    xk[bb] = *reinterpret_cast<const uint4*>(sk + 32 * bb);
    xv[bb] = *reinterpret_cast<const uint4*>(sv + 32 * bb);
  }
  const int pos = seq_len - 1;
  const int blk = a.bs_shift >= 0 ? (pos >> a.bs_shift) : (pos / L.bs);
  const int64_t prow = (int64_t)a.bt[(int64_t)b * a.max_blocks + blk] * L.bs + (pos - blk * L.bs);
#pragma unroll
  for (int i = lane; i < 256; i += 64) {
    if (i < nbk) s_t[0][i] = L.kt[i];
    if (i < nbv) s_t[1][i] = L.vt[i];
  }
  uint4 A[NB][2];
  tqq::hadamard_operands<NB>(L.signs, lane, A);
  float zero;  // an addend of 0 the compiler cannot fold, as in tq_quantize_kernel
  asm("v_mov_b32 %0, 0" : "=v"(zero));
  // the boundaries were written by other lanes of this wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint8_t* const dst = c == 0 ? a.pages_w + (prow * L.Hkv + h) * (int64_t)L.stride : tq_decode_append_discard;
  if (c == 0)  // padding, as the quantizer writes it (the discard buffer holds a plain slot only)
    for (int i = L.slot_bytes + g; i < L.stride; i += 4) dst[i] = 0;
  tqq::quantize_region<D, KB, false, false, false>(xk, A, zero, g, L.kcode_bytes, s_t[0], nullptr, 0,
                                                   nullptr, a.rsqrt_d, dst);
  tqq::quantize_region<D, VB, false, false, false>(xv, A, zero, g, L.vcode_bytes, s_t[1], nullptr, 0,
                                                   nullptr, a.rsqrt_d, dst + L.kreg);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the slot is stored
}

// QJL key format on the matrix cores: the residual term (S R q) . z of a 16-token sub-tile is one
// more product per 32 coordinates, A = the sketched query (two fp16 parts per head, rows as in
// QK), B = the tokens' sketch bits as fp16 +-1 (exact), four bits per read of a 16-entry table.
template <int D, int KB, int VB, bool G8, bool UBLK, bool QJL = false, bool MEANT = false>
__global__ __launch_bounds__(kWG, 2) void tq_decode_mfma_kernel(DecodeArgs a) {
  static_assert(!(QJL && UBLK), "the staged tile layout has no sketch");
  static_assert(!MEANT || UBLK, "MEANT: the staged tile layout of the mean-removal format");
  // Mean terms: on the per-lane path at run time, on the staged path in the MEANT instances only
  constexpr bool kMean = !UBLK || MEANT;
  using C = MfmaCfg<D, KB, VB>;
  using KE = typename OpTable<KB>::E;
  using VE = typename OpTable<VB>::E;
  using Tile = MfmaTile<D, KB, VB>;
  using Raw = MfmaRaw<D, KB, VB, MEANT>;
  constexpr int H8 = G8 ? 8 : 4;  // query heads per kv head this instance handles at most
  const TqLayer& L = a.L;
  const int G = L.G;

  // s_x holds, in turn: the rotated queries (prologue); per wave, the page rows of the current
  // tile (UBLK) or its value codes; the per-wave partial results (epilogue).  The fp16-row chunk
  // workgroups use it for their own sums.
  constexpr int kTileBytes = UBLK ? kNW * 32 * Raw::SS : kNW * 32 * C::VROW * 4;
  constexpr int kQPBytes = kNW * H8 * (D + 2) * 4;
  constexpr int kRowsBytes = G8 ? 0 : 4 * fp16_chunk_lds<D, 4>();
  constexpr int kXBytes = (kTileBytes > kQPBytes ? kTileBytes : kQPBytes) > kRowsBytes
                              ? (kTileBytes > kQPBytes ? kTileBytes : kQPBytes)
                              : kRowsBytes;
  __shared__ __align__(16) uint8_t s_x[kXBytes];
  if constexpr (!G8) {  // fp16-row chunks lead the grid (with 8 query heads: their own kernel)
    if ((int)blockIdx.x < a.rows_blocks) {
      fp16_chunk<D, 4>(a, blockIdx.x, reinterpret_cast<float*>(s_x));
      return;
    }
  }
  const int lin = blockIdx.x - a.rows_blocks;
  const int xcd = lin & 7;
  const int rest = lin >> 3;
  const int h = rest % L.Hkv;
  const int unit = (rest / L.Hkv) * 8 + xcd;
  if (unit >= a.n_units) return;
  const int b = unit / a.max_split;
  const int split = unit - b * a.max_split;
  const int tid = threadIdx.x;
  // Loads that do not need the sequence length are issued before it arrives: this thread's
  // codebook values for the operand tables, its query coordinates, and its entry of the block
  // table from block split * chunk on (the split's first block unless sinks move its start; the
  // entry is used only if it is).  All are in bounds: codes index their codebook, b < num_seqs,
  // and the entry is read only below max_blocks of a block table that is present.
  float kcv[OpTable<KB>::V], vcv[OpTable<VB>::V];
  load_op_values<KB>(L.kc, tid, kcv);
  load_op_values<VB>(L.vc, tid, vcv);
  constexpr int LPH = D / 8;
  uint4 qraw = make_uint4(0u, 0u, 0u, 0u);
  if (tid < LPH * G) qraw = *reinterpret_cast<const uint4*>(a.q + q_row(a, b, h, tid / LPH) * D + 8 * (tid % LPH));
  auto block_of = [&](int p) { return a.bs_shift >= 0 ? (p >> a.bs_shift) : (p / L.bs); };
  const int blk_pre = block_of(split * a.chunk);
  const bool bt_pre_ok = a.bt != nullptr && blk_pre + tid < a.max_blocks;
  const int32_t bt_pre = bt_pre_ok ? a.bt[(int64_t)b * a.max_blocks + blk_pre + tid] : 0;

  const int seq_len = a.seq_lens[b];
  const int ns = min(a.n_sink, seq_len);
  const int packed_end = seq_len - window_len(a, b, seq_len, ns);
  const int nsplit = num_splits(packed_end, a.chunk);
  if (split >= nsplit) return;

  __shared__ KE s_ktab[OpTable<KB>::N];
  __shared__ VE s_vtab[OpTable<VB>::N];
  __shared__ int64_t s_boff[kMaxBtLds];
  __shared__ float s_qmax[8];
  __shared__ float s_qsum[8];  // mean-removal format: scale log2(e) sum(q) per head
  __shared__ float s_r1[D];    // mean-removal format: R 1 = D^(-1/2) H s
  constexpr int NZ = D / 32;   // QJL products per 16-token sub-tile
  __shared__ __align__(16) uint4 s_ajq[QJL ? NZ : 1][64];  // QJL: A operands per step and lane
  __shared__ uint2 s_ztab[16];  // QJL: four sketch bits -> four fp16 +-1
  __shared__ float s_qjmax[8];  // QJL: largest |sketched query| per head, scaled
  __shared__ __align__(16) uint32_t s_w[kNW][16][C::WROW];
  constexpr bool kAppend = UBLK && !QJL && !MEANT;  // the fused append's instances
  __shared__ float s_app[kAppend ? 2 : 1][256];      // fused append: the boundaries
  float(*s_q)[D] = reinterpret_cast<float(*)[D]>(s_x);
  float(*s_qj)[D] = reinterpret_cast<float(*)[D]>(s_x) + 8;  // QJL: sketched queries, after s_q
  static_assert(!QJL || kXBytes >= 16 * D * 4, "room for the queries and the sketched queries");
  float(*s_part)[D + 2] = reinterpret_cast<float(*)[D + 2]>(s_x);  // [wave * H8 + head]

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t16 = lane & 15;
  const int q4 = lane >> 4;

  store_op_entry<KB>(s_ktab, kcv, tid);
  store_op_entry<VB>(s_vtab, vcv, tid);
  if (QJL && tid < 16) {  // entry e: fp16 +1 where bit i of e is set, else -1
    uint32_t hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = ((tid >> i) & 1) ? 0x3C00u : 0xBC00u;
    s_ztab[tid] = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
  }

  // The split's page positions start at the first non-sink one: the sinks' block-table entries
  // and page slots are never read (they may be absent).  The staged fetch needs 16-aligned runs,
  // so it starts at the run holding position ns, which lies in the block holding ns; rows below
  // ns are masked.  A split with no packed position reads nothing at all.
  const int p0 = max(split * a.chunk, UBLK ? (ns & ~15) : ns);
  const int p_end = min(split * a.chunk + a.chunk, packed_end);
  const bool any_rows = p_end > max(p0, ns);
  const int blk0 = any_rows ? block_of(p0) : 0;
  const int blk_last = any_rows ? block_of(p_end - 1) : blk0;
  const int nblk = any_rows ? blk_last - blk0 + 1 : 0;
  const int32_t* btg = a.bt + (int64_t)b * a.max_blocks + blk0;
  const int64_t row_bytes = (int64_t)L.Hkv * L.stride;
  for (int i = tid; i < nblk; i += kWG) {
    const int32_t e = (i == tid && blk0 == blk_pre && bt_pre_ok) ? bt_pre : btg[i];
    s_boff[i] = (int64_t)e * L.bs * row_bytes;
  }

  // Rotated queries H (s * q): D/8 lanes of one DPP row per head, 8 coordinates per lane; the
  // largest |q'| of each head sets its power-of-two scale into fp16 range below.
  if (tid < LPH * G) {
    const int g = tid / LPH, j = tid % LPH;
    float x[8];
    {
      const uint32_t w4[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = half_bits_to_float(w4[i] & 0xffffu);
        x[2 * i + 1] = half_bits_to_float(w4[i] >> 16);
      }
    }
    if (kMean && L.mean) {
      float qs = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) qs += x[e];
      qs = group_sum<LPH>(qs);
      if (j == 0) s_qsum[g] = qs * a.sink_scale;
    }
    const uint32_t sb = sign_byte(L.signs, j);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((sb >> e) & 1u) x[e] = -x[e];
    wht_row8_dpp<LPH>(x, j);
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_q[g][8 * j + e] = x[e];
      mx = fmaxf(mx, fabsf(x[e]));
    }
    mx = lanes_max<LPH>(mx);
    if (j == 0) s_qmax[g] = mx * a.qscale;
    if constexpr (QJL) {  // y = H (sigma2 * x); the score term is qscale sqrt(pi/2) / D y . z
      const uint32_t sb2 = sign_byte(L.signs2, j);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = ((sb2 >> e) & 1u) ? -x[e] : x[e];
      wht_row8_dpp<LPH>(y, j);
      float my = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s_qj[g][8 * j + e] = y[e];
        my = fmaxf(my, fabsf(y[e]));
      }
      my = lanes_max<LPH>(my);
      if (j == 0) s_qjmax[g] = my * a.qscale * (kQjlKappa / (float)D);
    }
  } else if (kMean && L.mean && tid >= 192 && tid < 192 + LPH) {  // R 1, by the last wave (G <= 8 heads
    const int j = tid - 192;                             // use at most 128 threads above)
    const uint32_t sb = sign_byte(L.signs, j);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = ((sb >> e) & 1u) ? -1.0f : 1.0f;
    wht_row8_dpp<LPH>(x, j);
#pragma unroll
    for (int e = 0; e < 8; ++e) s_r1[8 * j + e] = x[e] * a.rsqrt_d;
  }
  // Fused append: the last split of a sequence holds its new token's position.  Its last wave,
  // which the query rotation leaves idle (at most 8 heads of D / 8 lanes: the first two waves),
  // writes the token's slot of this kv head while the others rotate the queries; the stores are
  // complete before this barrier, which precedes every page load of the workgroup, so the
  // split's runs read the new slot (the same compute unit, the same L2).
  if constexpr (kAppend) {
    if (a.k_new != nullptr && seq_len > 0 && split == nsplit - 1 && wave == kNW - 1)
      append_row<D, KB, VB>(a, b, h, seq_len, lane, s_app);
  }
  __syncthreads();

  auto head_exp = [&](int g) {
    const float qm = s_qmax[g];
    return qm > 0.0f ? 13 - ilogbf(qm) : 0;
  };
  // A operand of QK, step st: coordinates QC q4 + 4 st + 0..3 of row m = t16 (one fp16 part),
  // repeated in the pattern of the key table.
  uint4 aq[C::NMQ];
  {
    const int g = (t16 >> 2) + 4 * ((t16 >> 1) & 1);
    const bool lo_part = t16 & 1;
    const bool live = g < G;
    const float f = live ? ldexpf(a.qscale, head_exp(g)) : 0.0f;
#pragma unroll
    for (int st = 0; st < C::NMQ; ++st) {
      uint32_t pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = live ? s_q[g][C::QC * q4 + 4 * st + i] * f : 0.0f;
        uint32_t hi, lo;
        split_f16(x, hi, lo);
        pr[i] = lo_part ? lo : hi;
      }
      aq[st] = repeat_operand<C::VK>(pr[0] | (pr[1] << 16), pr[2] | (pr[3] << 16));
    }
  }
  // QJL: A operands of the residual products, step st: coordinates QC q4 + 8 st + 0..7 of row
  // m = t16 (one fp16 part of qscale sqrt(pi/2) / D y, times the head's power of two).  They
  // depend on the lane only: wave 0 writes them for all waves.
  auto qj_exp = [&](int g) {
    const float qm = s_qjmax[g];
    return qm > 0.0f ? 13 - ilogbf(qm) : 0;
  };
  if constexpr (QJL) {
    if (wave == 0) {
      const int g = (t16 >> 2) + 4 * ((t16 >> 1) & 1);
      const bool lo_part = t16 & 1;
      const bool live = g < G;
      const float f = live ? ldexpf(a.qscale * (kQjlKappa / (float)D), qj_exp(g)) : 0.0f;
#pragma unroll
      for (int st = 0; st < NZ; ++st) {
        uint32_t pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = live ? s_qj[g][C::QC * q4 + 8 * st + i] * f : 0.0f;
          uint32_t hi, lo;
          split_f16(x, hi, lo);
          pr[i] = lo_part ? lo : hi;
        }
        s_ajq[st][lane] = make_uint4(pr[0] | (pr[1] << 16), pr[2] | (pr[3] << 16),
                                     pr[4] | (pr[5] << 16), pr[6] | (pr[7] << 16));
      }
    }
  }
  const int g0 = q4, g1 = q4 + 4;
  const bool live0 = g0 < G, live1 = G8 && g1 < G;
  // positions visible to heads g0, g1: the split's end, or earlier for causal queries
  const int lim0 = min(p_end, q_limit(a, seq_len, g0)), lim1 = min(p_end, q_limit(a, seq_len, g1));
  // Score factors of the heads this lane holds: 2^-(e + 8).
  const float f0 = live0 ? ldexpf(1.0f, -(head_exp(g0) + kLutShift)) : 0.0f;
  const float f1 = live1 ? ldexpf(1.0f, -(head_exp(g1) + kLutShift)) : 0.0f;
  // QJL: residual-term factors of the same heads, 2^-e
  const float fq0 = (QJL && live0) ? ldexpf(1.0f, -qj_exp(g0)) : 0.0f;
  const float fq1 = (QJL && live1) ? ldexpf(1.0f, -qj_exp(g1)) : 0.0f;

  const int voff = L.kreg;  // V region
  const uint32_t row_bytes32 = (uint32_t)row_bytes;
  const uint8_t* head_base = a.pages + (int64_t)h * L.stride;
  const int n_tiles = any_rows ? (p_end - p0 + 31) / 32 : 0;

  // Row base of the 16 positions starting at pu (a multiple of 16).  With a block size that is a
  // multiple of 16 the 16 rows lie in one page block, so the base is the same for the whole wave;
  // past the split's last position the last block is reused (rows in bounds, masked later).
  auto run_base = [&](int pu) {
    int bi = block_of(pu);
    int r0 = pu - bi * L.bs;
    if (bi > blk_last) {
      bi = blk_last;
      r0 = 0;
    }
    const int64_t boff = s_boff[bi - blk0];
    const int64_t o = (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(boff & 0xffffffff)) |
                      ((int64_t)__builtin_amdgcn_readfirstlane((int)(boff >> 32)) << 32);
    return head_base + o + (int64_t)r0 * row_bytes;
  };
  auto row_ptr = [&](int p) {  // any block size: one lane's row (masked rows re-read a packed one)
    const int pc = max(min(p, p_end - 1), p0);
    const int bi = block_of(pc);
    return head_base + s_boff[bi - blk0] + __umul24((uint32_t)(pc - bi * L.bs), row_bytes32);
  };
  // Blocks of any size: each lane loads the code runs and norms it works on (rows t16, 16 + t16).
  auto fetch = [&](int tile, Tile& m) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint8_t* r = row_ptr(p0 + 32 * tile + 16 * u + t16);
      load_words<C::KW>(r + 4 * C::KW * q4, m.k[u]);
      load_words<C::VW>(r + voff + 4 * C::VW * q4, m.v[u]);
      m.kn[u] = *reinterpret_cast<const float*>(r + L.kcode_bytes);
      m.vn[u] = *reinterpret_cast<const float*>(r + voff + L.vcode_bytes);
      m.km[u] = L.mean ? *reinterpret_cast<const float*>(r + L.kcode_bytes + 4) : 0.0f;
      m.vm[u] = L.mean ? *reinterpret_cast<const float*>(r + voff + L.vcode_bytes + 4) : 0.0f;
      if constexpr (QJL) {  // the lane group's QC sketch bits (4 or 2 bytes) and gamma
        if constexpr (C::QC == 32) m.zb[u] = *reinterpret_cast<const uint32_t*>(r + L.kqjl + 4 * q4);
        else m.zb[u] = *reinterpret_cast<const uint16_t*>(r + L.kqjl + 2 * q4);
        m.kg[u] = *reinterpret_cast<const float*>(r + L.kqjl + D / 8);
      }
    }
  };
  // Whole runs of 16 positions per block: the tile's slots as consecutive chunks (see MfmaRaw),
  // copied into the wave's stage (slot of row r at r * SB; SB / 4 = 2 mod 4, so the code runs of
  // 16 consecutive rows, and the value codes of rows t and t + 8, fall on distinct banks).
  constexpr int kFull = 32 * Raw::N16;  // chunks in a tile
  uint32_t goff[Raw::NI], loff[Raw::NI];
#pragma unroll
  for (int i = 0; i < Raw::NI; ++i) {
    const int c = 64 * i + lane;
    const int row = c / Raw::N16, col = c - row * Raw::N16;
    goff[i] = __umul24((uint32_t)(row & 15), row_bytes32) + 16 * col;
    loff[i] = row * Raw::SS + 16 * col;
  }
  const uint32_t goff_t = __umul24((uint32_t)(lane & 15), row_bytes32) + 16 * Raw::N16;
  auto fetch_raw = [&](int tile, Raw& m) {
    const int pu = p0 + 32 * tile;
    const uint8_t* r0 = run_base(pu);
    const uint8_t* r1 = run_base(pu + 16);
#pragma unroll
    for (int i = 0; i < Raw::NI; ++i) {
      const int clo = 64 * i, chi = 64 * i + 63;
      if (chi < kFull || lane + clo < kFull) {
        const uint8_t* base = chi / Raw::N16 < 16 ? r0
                              : clo / Raw::N16 >= 16 ? r1
                              : ((lane + clo) / Raw::N16 < 16 ? r0 : r1);
        m.c[i] = *reinterpret_cast<const uint4*>(base + goff[i]);
      }
    }
    if (Raw::TAIL && lane < 32) m.t = *reinterpret_cast<const uint2*>((lane < 16 ? r0 : r1) + goff_t);
  };
  uint8_t* stage = s_x + wave * 32 * Raw::SS;
  auto stage_raw = [&](const Raw& m) {
#pragma unroll
    for (int i = 0; i < Raw::NI; ++i) {
      if (64 * i + 63 < kFull || lane + 64 * i < kFull) {
        uint2* d = reinterpret_cast<uint2*>(stage + loff[i]);
        d[0] = make_uint2(m.c[i].x, m.c[i].y);
        d[1] = make_uint2(m.c[i].z, m.c[i].w);
      }
    }
    if (Raw::TAIL && lane < 32) *reinterpret_cast<uint2*>(stage + lane * Raw::SS + 16 * Raw::N16) = m.t;
  };

  // Online-softmax state.  kSent is a finite "minus infinity": masked positions score kSent, so
  // no exp2 ever sees -inf - -inf; anything accumulated while the maximum is still kSent is
  // scaled by exp2(kSent - m) = 0 as soon as a real score arrives.
  float m_s[2] = {kSent, kSent};   // running max of scores (heads g0, g1)
  float m_w[2] = {kSent, kSent};   // running max of score + log2(n_V)
  float l_s[2] = {0.0f, 0.0f};     // per-lane partial sums of 2^(s - m_s)
  float mv_s[2] = {0.0f, 0.0f};    // mean-removal format: partial sums of 2^(s - m_s) mu_V
  const float qsum0 = (kMean && L.mean && live0) ? s_qsum[g0] : 0.0f;  // mu_K term of the scores
  const float qsum1 = (kMean && L.mean && live1) ? s_qsum[g1] : 0.0f;
  float4_t acc[C::PC];
#pragma unroll
  for (int c = 0; c < C::PC; ++c) acc[c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  uint32_t* wt = &s_w[wave][0][0];
  uint32_t* vt = reinterpret_cast<uint32_t*>(s_x) + wave * 32 * C::VROW;  // value codes (!UBLK)
  uint16_t* wt16 = reinterpret_cast<uint16_t*>(wt);
  // weight of row m, token col: a fp16 at [m][col], or the pair (w, w) at dword [m][col]
  auto put_w = [&](int m, int col, uint32_t w) {
    if constexpr (C::VV == 1) wt[m * C::WROW + col] = w | (w << 16);
    else wt16[m * 2 * C::WROW + col] = (uint16_t)w;
  };
  if (!G8) {  // weight rows of heads 4..7 stay zero
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      put_w(4 * q4 + 2, 16 * u + t16, 0);
      put_w(4 * q4 + 3, 16 * u + t16, 0);
    }
  }
  __syncthreads();  // tables, block offsets, zero rows ready

  // cur: the lane's code runs and norms (blocks of any size); with UBLK they come from the stage.
  auto process = [&](const Tile& cur, int tile) {
    // ---- QK on the matrix cores ----
    float4_t sc[2], sq[2];
    float kn[2], vn[2], km[2] = {0.0f, 0.0f}, vm[2] = {0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t kw[C::KW];
      if constexpr (UBLK) {
        const uint8_t* row = stage + (16 * u + t16) * Raw::SS;
        if constexpr (C::KW % 2 == 0) {
#pragma unroll
          for (int i = 0; i < C::KW; i += 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(row + 4 * C::KW * q4 + 4 * i);
            kw[i] = x.x;
            kw[i + 1] = x.y;
          }
        } else {
#pragma unroll
          for (int i = 0; i < C::KW; ++i) kw[i] = reinterpret_cast<const uint32_t*>(row + 4 * C::KW * q4)[i];
        }
        kn[u] = *reinterpret_cast<const float*>(row + L.kcode_bytes);
        vn[u] = *reinterpret_cast<const float*>(row + voff + L.vcode_bytes);
        if constexpr (MEANT) {  // the row means follow the norms
          km[u] = *reinterpret_cast<const float*>(row + L.kcode_bytes + 4);
          vm[u] = *reinterpret_cast<const float*>(row + voff + L.vcode_bytes + 4);
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::KW; ++i) kw[i] = cur.k[u][i];
        kn[u] = cur.kn[u];
        vn[u] = cur.vn[u];
        km[u] = cur.km[u];
        vm[u] = cur.vm[u];
      }
      uint4 kop[C::NMQ];  // all table reads of the sub-tile first, so their latency overlaps
#pragma unroll
      for (int st = 0; st < C::NMQ; ++st) kop[st] = k_operand<KB>(s_ktab, kw, st);
      float4_t sa = float4_t{0.0f, 0.0f, 0.0f, 0.0f}, sb = sa;  // two independent MFMA chains
#pragma unroll
      for (int st = 0; st < C::NMQ; st += 2) {
        sa = mfma_f16(aq[st], kop[st], sa);
        sb = mfma_f16(aq[st + 1], kop[st + 1], sb);
      }
      sc[u] = sa + sb;
      if constexpr (QJL) {  // residual products: sketch bits as fp16 +-1, four per table read
        float4_t za = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < NZ; ++st) {
          const uint32_t byte = (cur.zb[u] >> (8 * st)) & 0xffu;
          const uint2 lo = s_ztab[byte & 15u], hi = s_ztab[byte >> 4];
          za = mfma_f16(s_ajq[st][lane], make_uint4(lo.x, lo.y, hi.x, hi.y), za);
        }
        sq[u] = za;
      }
    }

    // ---- online softmax, tokens t16 and 16 + t16 ----
    const int pbase = p0 + 32 * tile;
    float s0[2], s1[2], lv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int p = pbase + 16 * u + t16;
      float t0 = (sc[u][0] + sc[u][1]) * kn[u] * f0, t1 = (sc[u][2] + sc[u][3]) * kn[u] * f1;
      if constexpr (QJL) {
        t0 += (sq[u][0] + sq[u][1]) * cur.kg[u] * fq0;
        t1 += (sq[u][2] + sq[u][3]) * cur.kg[u] * fq1;
      }
      if constexpr (kMean) {
        t0 += km[u] * qsum0;
        t1 += km[u] * qsum1;
      }
      s0[u] = (p >= ns && p < lim0 && live0) ? t0 : kSent;
      if (G8) s1[u] = (p >= ns && p < lim1 && live1) ? t1 : kSent;
      // log2(n_V) (-inf for a zero row).  Rows outside [ns, p_end) are not packed tokens of this
      // split (sink or hot-window slots, slots not yet written): whatever bytes they hold, they
      // add nothing, neither to the weights' maximum nor to the mean sums.
      const bool packed = p >= ns && p < p_end;
      lv[u] = packed ? __builtin_amdgcn_logf(vn[u]) : 0.0f;
      if constexpr (kMean) vm[u] = packed ? vm[u] : 0.0f;
    }
    const float ms0 = fmaxf(m_s[0], row16_max(fmaxf(s0[0], s0[1])));
    const float mw0 = fmaxf(m_w[0], row16_max(fmaxf(s0[0] + lv[0], s0[1] + lv[1])));
    float ms1 = kSent, mw1 = kSent;
    if (G8) {
      ms1 = fmaxf(m_s[1], row16_max(fmaxf(s1[0], s1[1])));
      mw1 = fmaxf(m_w[1], row16_max(fmaxf(s1[0] + lv[0], s1[1] + lv[1])));
    }
    if (ms0 > m_s[0]) {
      const float r = __builtin_amdgcn_exp2f(m_s[0] - ms0);
      l_s[0] *= r;
      if constexpr (kMean) mv_s[0] *= r;
    }
    m_s[0] = ms0;
    if (G8) {
      if (ms1 > m_s[1]) {
        const float r = __builtin_amdgcn_exp2f(m_s[1] - ms1);
        l_s[1] *= r;
        if constexpr (kMean) mv_s[1] *= r;
      }
      m_s[1] = ms1;
    }
    const bool grow0 = mw0 > m_w[0], grow1 = G8 && mw1 > m_w[1];
    if (grow0 || grow1) {
      const float r0 = grow0 ? __builtin_amdgcn_exp2f(m_w[0] - mw0) : 1.0f;
      const float r1 = grow1 ? __builtin_amdgcn_exp2f(m_w[1] - mw1) : 1.0f;
#pragma unroll
      for (int c = 0; c < C::PC; ++c) {
        acc[c][0] *= r0;
        acc[c][1] *= r0;
        if (G8) {
          acc[c][2] *= r1;
          acc[c][3] *= r1;
        }
      }
    }
    m_w[0] = mw0;
    if (G8) m_w[1] = mw1;
    // weights enter the product scaled by 2^kWShift: fold the shift into the reference maximum
    const float mw0s = mw0 - (float)kWShift, mw1s = mw1 - (float)kWShift;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // last tile's tile reads are done
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int col = 16 * u + t16;
      const float p0 = __builtin_amdgcn_exp2f(s0[u] - ms0);
      l_s[0] += p0;
      if constexpr (kMean) mv_s[0] += p0 * vm[u];
      uint32_t h0, l0;
      split_f16(__builtin_amdgcn_exp2f(s0[u] + lv[u] - mw0s), h0, l0);
      put_w(4 * q4 + 0, col, h0);
      put_w(4 * q4 + 1, col, l0);
      if (G8) {
        const float p1 = __builtin_amdgcn_exp2f(s1[u] - ms1);
        l_s[1] += p1;
        if constexpr (kMean) mv_s[1] += p1 * vm[u];
        uint32_t h1, l1;
        split_f16(__builtin_amdgcn_exp2f(s1[u] + lv[u] - mw1s), h1, l1);
        put_w(4 * q4 + 2, col, h1);
        put_w(4 * q4 + 3, col, l1);
      }
      if constexpr (!UBLK) {  // value codes of token col, lane group q4's run of coordinates
        uint32_t* vrow = vt + col * C::VROW + C::VW * q4;
#pragma unroll
        for (int i = 0; i < C::VW; i += 2)
          *reinterpret_cast<uint2*>(vrow + i) = make_uint2(cur.v[u][i], cur.v[u][i + 1]);
      }
    }

    // ---- PV on the matrix cores: lane (n = t16, q4) handles tokens 8 q4 .. 8 q4 + 7 and
    // coordinates PC t16 .. PC t16 + PC - 1 (MFMA c covers coordinate PC n + c of column n) ----
    // The tiles written above are read back by other lanes of this wave: order the LDS accesses.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    constexpr int VBITS = C::PC * VB;  // code bits of the lane's coordinates per token (8..64)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // weights of tokens 8 q4 + 4 j + 0..3 of row t16, in the pattern of the value table
      uint4 aw;
      if constexpr (C::VV == 1) {
        aw = *reinterpret_cast<const uint4*>(wt + t16 * C::WROW + 8 * q4 + 4 * j);
      } else {
        const uint32_t* wrow = wt + t16 * C::WROW + 4 * q4 + 2 * j;
        aw = repeat_operand<C::VV>(wrow[0], wrow[1]);
      }
      // codes of the lane's coordinates for the four tokens 8 q4 + 4 j + i
      uint32_t cw[4][VBITS > 32 ? 2 : 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 8 * q4 + 4 * j + i;
        const uint32_t* src = UBLK ? reinterpret_cast<const uint32_t*>(stage + tok * Raw::SS + voff)
                                   : vt + tok * C::VROW;
        if constexpr (VBITS == 64) {  // the stage's value codes are 4-byte aligned only
          cw[i][0] = src[2 * t16];
          cw[i][1] = src[2 * t16 + 1];
        } else if constexpr (VBITS == 32) {
          cw[i][0] = src[t16];
        } else if constexpr (VBITS == 16) {
          cw[i][0] = reinterpret_cast<const uint16_t*>(src)[t16];
        } else {
          cw[i][0] = reinterpret_cast<const uint8_t*>(src)[t16];
        }
      }
      uint4 vop[C::PC];
      if constexpr (VB == 8) {
        // one byte per (token, coordinate): four single-value reads per operand
#pragma unroll
        for (int c = 0; c < C::PC; ++c) {
          const int wi = c >> 2, sh = 8 * (c & 3);
          vop[c] = make_uint4(s_vtab[(cw[0][wi] >> sh) & 0xffu], s_vtab[(cw[1][wi] >> sh) & 0xffu],
                              s_vtab[(cw[2][wi] >> sh) & 0xffu], s_vtab[(cw[3][wi] >> sh) & 0xffu]);
        }
      } else if constexpr (VB == 4) {
        // E, O: bytes (nibble c of token 2i, nibble c of token 2i + 1) for even / odd c
        uint32_t eo[2][2];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const uint32_t x = cw[2 * pr][0], y = cw[2 * pr + 1][0];
          eo[pr][0] = (x & 0x0f0f0f0fu) | ((y << 4) & 0xf0f0f0f0u);
          eo[pr][1] = ((x >> 4) & 0x0f0f0f0fu) | (y & 0xf0f0f0f0u);
        }
#pragma unroll
        for (int c = 0; c < C::PC; ++c) {
          const uint32_t sh = 8 * (c >> 1);
          const uint2 e0 = s_vtab[(eo[0][c & 1] >> sh) & 0xffu];
          const uint2 e1 = s_vtab[(eo[1][c & 1] >> sh) & 0xffu];
          vop[c] = make_uint4(e0.x, e0.y, e1.x, e1.y);
        }
      } else {
        // VB == 2: bytes (code c of tokens 0, 1, 2, 3 at bits 0, 2, 4, 6) for the 8 coordinates
        uint32_t pe[2], po[2];  // token pairs (0,1), (2,3): nibbles (code a, code b), even / odd c
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const uint32_t x = cw[2 * pr][0], y = cw[2 * pr + 1][0];
          pe[pr] = (x & 0x3333u) | ((y & 0x3333u) << 2);
          po[pr] = ((x >> 2) & 0x3333u) | (y & 0xccccu);
        }
        // nibble k of pe = coordinate 2k, of po = coordinate 2k + 1
        const uint32_t r0 = (pe[0] & 0x0f0fu) | ((pe[1] & 0x0f0fu) << 4);          // c = 0, 4
        const uint32_t r1 = (po[0] & 0x0f0fu) | ((po[1] & 0x0f0fu) << 4);          // c = 1, 5
        const uint32_t r2 = ((pe[0] >> 4) & 0x0f0fu) | (pe[1] & 0xf0f0u);          // c = 2, 6
        const uint32_t r3 = ((po[0] >> 4) & 0x0f0fu) | (po[1] & 0xf0f0u);          // c = 3, 7
        const uint32_t rr[4] = {r0, r1, r2, r3};
#pragma unroll
        for (int c = 0; c < C::PC; ++c) vop[c] = s_vtab[(rr[c & 3] >> (8 * (c >> 2))) & 0xffu];
      }
#pragma unroll
      for (int c = 0; c < C::PC; ++c) acc[c] = mfma_f16(aw, vop[c], acc[c]);
    }
  };

  if constexpr (UBLK) {
    Raw raw;  // the next tile in flight while the stage holds the current one
    if (wave < n_tiles) fetch_raw(wave, raw);
    for (int tile = wave; tile < n_tiles; tile += kNW) {
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // last tile's stage reads are done
      stage_raw(raw);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // stage written: read by other lanes
      if (tile + kNW < n_tiles) fetch_raw(tile + kNW, raw);
      process(Tile{}, tile);
    }
  } else {
    Tile cur;
    if (wave < n_tiles) fetch(wave, cur);
    for (int tile = wave; tile < n_tiles; tile += kNW) {
      Tile nxt;
      if (tile + kNW < n_tiles) fetch(tile + kNW, nxt);
      process(cur, tile);
      cur = nxt;
    }
  }
  __syncthreads();  // every wave is done with s_x: it takes the partial results

  // ---- wave result: heads g0, g1 at coordinates PC t16 + c, in the score-max frame ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    l_s[i] += dpp<kDppQuadXor1>(l_s[i]);
    l_s[i] += dpp<kDppQuadXor2>(l_s[i]);
    l_s[i] += dpp<kDppHalfRowMirror>(l_s[i]);
    l_s[i] += dpp<kDppRowMirror>(l_s[i]);
    if constexpr (kMean) {
      mv_s[i] += dpp<kDppQuadXor1>(mv_s[i]);
      mv_s[i] += dpp<kDppQuadXor2>(mv_s[i]);
      mv_s[i] += dpp<kDppHalfRowMirror>(mv_s[i]);
      mv_s[i] += dpp<kDppRowMirror>(mv_s[i]);
    }
  }
  const float vscale = ldexpf(1.0f, -(kWShift + kLutShift));
  const float c0 = __builtin_amdgcn_exp2f(m_w[0] - m_s[0]) * vscale;
  const float c1 = __builtin_amdgcn_exp2f(m_w[1] - m_s[1]) * vscale;
  // mean-removal format: the weighted means sum_p w_p mu_p enter the rotated accumulator as
  // (sum) R 1, which the merge's R^T turns into (sum) 1
  auto mean_term = [&](int i, int c) { return kMean && L.mean ? mv_s[i] * s_r1[C::PC * t16 + c] : 0.0f; };
  if (live0) {
#pragma unroll
    for (int c = 0; c < C::PC; ++c)
      s_part[wave * H8 + g0][2 + C::PC * t16 + c] = (acc[c][0] + acc[c][1]) * c0 + mean_term(0, c);
    if (t16 == 0) {
      s_part[wave * H8 + g0][0] = m_s[0];
      s_part[wave * H8 + g0][1] = l_s[0];
    }
  }
  if (live1) {
#pragma unroll
    for (int c = 0; c < C::PC; ++c)
      s_part[wave * H8 + g1][2 + C::PC * t16 + c] = (acc[c][2] + acc[c][3]) * c1 + mean_term(1, c);
    if (t16 == 0) {
      s_part[wave * H8 + g1][0] = m_s[1];
      s_part[wave * H8 + g1][1] = l_s[1];
    }
  }
  __syncthreads();

  const int64_t bh = (int64_t)b * L.Hkv + h;
  float* part = a.partials + (bh * a.part_stride + split) * (int64_t)G * (D + 2);
  for (int i = tid; i < G * (D + 2); i += kWG) {
    const int g = i / (D + 2), d = i % (D + 2);
    float M = kSent;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_part[w * H8 + g][0]);
    float r;
    if (d == 0) {
      r = M;
    } else {
      r = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w)
        r += s_part[w * H8 + g][d] * __builtin_amdgcn_exp2f(s_part[w * H8 + g][0] - M);
    }
    part[i] = r;
  }
}

// Fold NB loaded partials (ms, ls, as: maximum, sum, coordinate d) into the running (M, l, acc).
template <int NB>
__device__ __forceinline__ void merge_fold(const float (&ms)[NB], const float (&ls)[NB], const float (&as)[NB],
                                           float& M, float& l, float& acc) {
  float mc = ms[0];
#pragma unroll
  for (int k = 1; k < NB; ++k) mc = fmaxf(mc, ms[k]);
  const float Mn = fmaxf(M, mc);
  const float fo = __builtin_amdgcn_exp2f(M - Mn);
  l *= fo;
  acc *= fo;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const float fn = __builtin_amdgcn_exp2f(ms[k] - Mn);
    l += ls[k] * fn;
    acc += as[k] * fn;
  }
  M = Mn;
}

// NB partials from index s0 into the running (M, l, acc) of coordinate d.
template <int NB, int D>
__device__ __forceinline__ void merge_batch(const DecodeArgs& a, const float* pb, int s0, int nparts, int nsplit,
                                            int G, int d, float& M, float& l, float& acc) {
  float ms[NB], ls[NB], as[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int pi = s0 + k;
    const bool in = pi < nparts;
    const int idx = !in ? 0 : pi < nsplit ? pi : a.max_split + (pi - nsplit);
    const float* e = pb + (int64_t)idx * G * (D + 2);
    ms[k] = in ? e[0] : -INFINITY;
    ls[k] = in ? e[1] : 0.0f;
    as[k] = in ? e[2 + d] : 0.0f;
  }
  merge_fold<NB>(ms, ls, as, M, l, acc);
}

// One workgroup per (sequence, kv head, query head), one thread per coordinate: merge the packed
// splits and the fp16-row chunks, rotate back, normalise.
// PRE: partials whose loads are issued before the sequence's partial count is known (16 when the
// launch expects about sixteen per sequence, else 4).
template <int D, int GMAX, int PRE>
__global__ __launch_bounds__(D) void tq_decode_merge_kernel(DecodeArgs a) {
  const TqLayer& L = a.L;
  const int G = L.G;
  const int g = blockIdx.x % G;
  const int bh = blockIdx.x / G;
  const int h = bh % L.Hkv;
  const int b = bh / L.Hkv;
  const int d = threadIdx.x;
  const float* pb = a.partials + (int64_t)bh * a.part_stride * G * (D + 2) + g * (D + 2);
  // Without fp16 rows in the call the first partials are packed splits at indices 0..PRE-1: their
  // loads go out with those of the sequence's length and partial count instead of after them
  // (indices past the stride are clamped into this row of partials and masked below).
  constexpr int kPre = PRE;
  float pm[kPre], pl[kPre], pa[kPre];
  const bool pre = a.row_chunks == 0;
  if (pre) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const float* e = pb + (int64_t)min(k, a.part_stride - 1) * G * (D + 2);
      pm[k] = e[0];
      pl[k] = e[1];
      pa[k] = e[2 + d];
    }
  }
  const int seq_len = a.seq_lens[b];
  if (seq_len == 0) {
    a.out[q_row(a, b, h, g) * D + d] = 0.0f;
    return;
  }
  const int nf = fp16_rows(a, b, seq_len);
  const int nsplit = a.nsplit_of != nullptr ? a.nsplit_of[b]
                                             : num_splits(seq_len - (nf - min(a.n_sink, seq_len)), a.chunk);
  const int nrc = (nf + kRowChunk - 1) / kRowChunk;
  const int nparts = nsplit + nrc;
  __shared__ float s_acc[D];  // merged rotated accumulator

  // Log-sum-exp merge of the partials (packed splits, then fp16-row chunks), sixteen at a time so
  // their loads are in flight together, the rest four at a time.  Empty partials carry a maximum
  // of -inf or kSent and contribute exp2(. - M) = 0 once a real score is in M.
  float M = kSent, l = 0.0f, acc = 0.0f;
  int s0 = 0;
  if (pre) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const bool in = k < nparts;
      pm[k] = in ? pm[k] : -INFINITY;
      pl[k] = in ? pl[k] : 0.0f;
      pa[k] = in ? pa[k] : 0.0f;
    }
    merge_fold<kPre>(pm, pl, pa, M, l, acc);
    s0 = kPre;
  }
  for (; s0 + 16 <= nparts; s0 += 16) merge_batch<16, D>(a, pb, s0, nparts, nsplit, G, d, M, l, acc);
  for (; s0 < nparts; s0 += 4) merge_batch<4, D>(a, pb, s0, nparts, nsplit, G, d, M, l, acc);
  s_acc[d] = acc;
  __syncthreads();

  // R^T a = D^(-1/2) diag(s) H a, divided by the sum: D/8 lanes of one DPP row, 8 coordinates each.
  constexpr int LPH = D / 8;
  if (d < LPH) {
    const int j = d;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s_acc[8 * j + e];
    wht_row8_dpp<LPH>(x, j);
    const uint32_t sb = sign_byte(L.signs, j);
    // a query before the first position (several queries per sequence) sees nothing: zero
    const float inv_l = q_limit(a, seq_len, g) > 0 ? 1.0f / l : 0.0f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = x[e] * a.rsqrt_d;
      if ((sb >> e) & 1u) o[e] = -o[e];
    }
    float4* o4 = reinterpret_cast<float4*>(a.out + q_row(a, b, h, g) * D + 8 * j);
    o4[0] = make_float4(o[0] * inv_l, o[1] * inv_l, o[2] * inv_l, o[3] * inv_l);
    o4[1] = make_float4(o[4] * inv_l, o[5] * inv_l, o[6] * inv_l, o[7] * inv_l);
  }
}

// fp16-row chunks on their own (for the split kernel whose LDS budget leaves no room for them).
template <int D, int GMAX>
__global__ __launch_bounds__(kWG) void tq_decode_rows_kernel(DecodeArgs a) {
  __shared__ float s_rows[fp16_chunk_lds<D, GMAX>()];
  fp16_chunk<D, GMAX>(a, blockIdx.x, s_rows);
}

template <int D, int GMAX>
void launch_merge(const DecodeArgs& a, dim3 mgrid, hipStream_t st) {
  if (a.merge_pre >= 12) hipLaunchKernelGGL((tq_decode_merge_kernel<D, GMAX, 16>), mgrid, dim3(D), 0, st, a);
  else hipLaunchKernelGGL((tq_decode_merge_kernel<D, GMAX, 4>), mgrid, dim3(D), 0, st, a);
}

// Split kernel for one format and query-group bound (the fp16-row chunks at the front of its grid,
// or in a kernel of their own before it), then the merge.  `grid` holds the packed splits only;
// a.rows_blocks is the number of fp16-row chunk workgroups.
template <int D, int KB, int VB, int GMAX>
void launch_t(const DecodeArgs& a0, dim3 sgrid, dim3 mgrid, hipStream_t st) {
  DecodeArgs a = a0;
  constexpr bool separate_rows = mfma_format(D, KB, VB) && GMAX > 4;
  dim3 grid = sgrid;
  if (separate_rows) {
    if (a.rows_blocks > 0)
      hipLaunchKernelGGL((tq_decode_rows_kernel<D, GMAX>), dim3(a.rows_blocks), dim3(kWG), 0, st, a);
    a.rows_blocks = 0;
  } else {
    grid.x += a.rows_blocks;
  }
  // The QJL key format (keys of 2-4 bits) has its own instances: the matrix-core kernel with the
  // residual products, or the vector kernel with the residual term.
  constexpr bool kQjlOk = KB <= 4;
  if constexpr (mfma_format(D, KB, VB)) {
    constexpr bool G8 = GMAX > 4;
    if (kQjlOk && a.L.qjl)
      hipLaunchKernelGGL((tq_decode_mfma_kernel<D, KB, VB, G8, false, kQjlOk>), grid, dim3(kWG), 0, st, a);
    else if (a.L.bs % 16 == 0 && !a.L.mean)  // staged tiles (whole runs of 16 rows per block)
      hipLaunchKernelGGL((tq_decode_mfma_kernel<D, KB, VB, G8, true>), grid, dim3(kWG), 0, st, a);
    else if (a.L.bs % 16 == 0)  // staged tiles of the mean-removal format
      hipLaunchKernelGGL((tq_decode_mfma_kernel<D, KB, VB, G8, true, false, true>), grid, dim3(kWG), 0, st, a);
    else
      hipLaunchKernelGGL((tq_decode_mfma_kernel<D, KB, VB, G8, false>), grid, dim3(kWG), 0, st, a);
  } else {
    if (kQjlOk && a.L.qjl)
      hipLaunchKernelGGL((tq_decode_split_kernel<D, KB, VB, GMAX, kQjlOk>), grid, dim3(kWG), 0, st, a);
    else
      hipLaunchKernelGGL((tq_decode_split_kernel<D, KB, VB, GMAX>), grid, dim3(kWG), 0, st, a);
  }
  launch_merge<D, GMAX>(a, mgrid, st);
}

template <int D, int KB, int VB>
void launch_g(const DecodeArgs& a, dim3 grid, dim3 mgrid, hipStream_t st) {
  const int G = a.L.G;
  if constexpr (mfma_format(D, KB, VB)) {  // the matrix-core kernel covers G <= 4 in one instance
    if (G <= 4) launch_t<D, KB, VB, 4>(a, grid, mgrid, st);
    else launch_t<D, KB, VB, 8>(a, grid, mgrid, st);
  } else {
    if (G <= 1) launch_t<D, KB, VB, 1>(a, grid, mgrid, st);
    else if (G <= 2) launch_t<D, KB, VB, 2>(a, grid, mgrid, st);
    else if (G <= 4) launch_t<D, KB, VB, 4>(a, grid, mgrid, st);
    else launch_t<D, KB, VB, 8>(a, grid, mgrid, st);
  }
}

template <int D, int KB>
void launch_v(const DecodeArgs& a, dim3 grid, dim3 mgrid, hipStream_t st) {
  switch (a.L.vb) {
    case 2: launch_g<D, KB, 2>(a, grid, mgrid, st); break;
    case 3: launch_g<D, KB, 3>(a, grid, mgrid, st); break;
    case 4: launch_g<D, KB, 4>(a, grid, mgrid, st); break;
    default: launch_g<D, KB, 8>(a, grid, mgrid, st); break;
  }
}

template <int D>
void launch_k(const DecodeArgs& a, dim3 grid, dim3 mgrid, hipStream_t st) {
  switch (a.L.kb) {
    case 2: launch_v<D, 2>(a, grid, mgrid, st); break;
    case 3: launch_v<D, 3>(a, grid, mgrid, st); break;
    case 4: launch_v<D, 4>(a, grid, mgrid, st); break;
    default: launch_v<D, 8>(a, grid, mgrid, st); break;
  }
}

int ilog2_exact(int v) {
  for (int s = 0; s < 31; ++s)
    if ((1 << s) == v) return s;
  return -1;
}

}  // namespace

// Formats whose decode call also takes the step's append (tq_paged_decode_attention_append):
// plain slots (no norm correction, mean or sketch) of the block kernel's formats, or of the
// matrix-core split kernel's formats with page blocks of whole 16-position runs (its staged
// instances).
bool tq_decode_append_format(const TqLayer& L) {
  if (L.norm_corr || L.mean || L.qjl) return false;
  return tq_decode_block_format(L) || (mfma_format(L.D, L.kb, L.vb) && L.bs % 16 == 0);
}

// Split geometry: page tokens per split are a multiple of 32 (the tokens a workgroup covers per
// step) and span at most kMaxBtLds page blocks.  About three workgroups per CU: each workgroup
// pays a fixed prologue (rotated query, lookup tables, block offsets) and writes one partial, so
// fewer, longer splits win as long as every CU still holds a few of them.
TqSplit tq_decode_split(const TqLayer& L, int num_seqs, int max_seq_len) {
  if (tq_decode_block_format(L)) return tq_decode_block_split(num_seqs, max_seq_len);
  const long bh = (long)num_seqs * L.Hkv;
  const long tokens = (long)(max_seq_len > 0 ? max_seq_len : 1);
  const long target_wgs = 768;
  long chunk = (tokens * bh + target_wgs - 1) / target_wgs;
  if (chunk < 256) chunk = 256;
  if (chunk > 16384) chunk = 16384;
  const long bt_cap = ((long)(kMaxBtLds - 2) * L.bs / 32) * 32;  // blocks a split may touch
  if (chunk > bt_cap) chunk = bt_cap;
  chunk = ((chunk + 31) / 32) * 32;
  TqSplit sp;
  sp.chunk = (int)chunk;
  sp.max_split = (int)((tokens + chunk - 1) / chunk);
  if (sp.max_split < 1) sp.max_split = 1;
  return sp;
}

// Partials per (sequence, kv head): the packed splits, then one per chunk of fp16 rows (sinks and
// hot-window rows) of this call.
static int row_chunks_of(int n_sink, int win_cap) { return (n_sink + win_cap + kRowChunk - 1) / kRowChunk; }

// Partials, then (block kernel) the piece count of each sequence.
static size_t partials_bytes(const TqLayer& L, int num_seqs, const TqSplit& sp, int n_sink, int win_cap) {
  const size_t bh = (size_t)num_seqs * L.Hkv;
  const size_t b = bh * (size_t)(sp.max_split + row_chunks_of(n_sink, win_cap)) * L.G * (L.D + 2) * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

size_t tq_decode_ws_bytes_for(const TqLayer& L, int num_seqs, const TqSplit& sp, int n_sink, int win_cap) {
  const size_t meta = tq_decode_block_format(L) ? (size_t)num_seqs * sizeof(int32_t) : 0;
  return partials_bytes(L, num_seqs, sp, n_sink, win_cap) + meta;
}

size_t tq_decode_ws_bytes(const TqLayer& L, int num_seqs, const TqSplit& sp) {
  // room for the fp16-row chunks of the largest sink count and window
  return tq_decode_ws_bytes_for(L, num_seqs, sp, TQ_MAX_SINKS, TQ_MAX_WINDOW);
}

// The split-K partials of tq_paged_decode_attention_noalloc, for callers that cannot allocate:
// one array per GPU, loaded with the library and held until the process ends.  Host code reaches
// it only through the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_WORKSPACE_BYTES];

int tq_noalloc_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *ptr = ptrs[dev];
  return 0;
}

int tq_launch_decode(const TqLayer& L, const void* q, const void* pages, const int32_t* block_tables,
                     int max_blocks, const int32_t* seq_lens, int num_seqs, const TqSplit& sp,
                     const void* sink_k, const void* sink_v, int n_sink, const void* win_k,
                     const void* win_v, const int32_t* win_lens, int win_cap, float scale,
                     float* out, void* workspace, void* stream, int nq, int q0, int g_real,
                     const TqAppend* app) {
  if (num_seqs == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  DecodeArgs a;
  a.L = L;
  a.rsqrt_d = (float)(1.0 / __builtin_sqrt((double)L.D));
  a.qscale = scale * kLog2e * a.rsqrt_d;
  a.sink_scale = scale * kLog2e;
  a.q = (const uint16_t*)q;
  a.pages = (const uint8_t*)pages;
  a.bt = block_tables;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.chunk = sp.chunk;
  a.max_split = sp.max_split;
  a.row_chunks = row_chunks_of(n_sink, win_cap);
  a.part_stride = sp.max_split + a.row_chunks;
  a.rows_blocks = num_seqs * L.Hkv * a.row_chunks;
  a.n_units = num_seqs * sp.max_split;
  a.bs_shift = ilog2_exact(L.bs);
  a.sink_k = (const uint16_t*)sink_k;
  a.sink_v = (const uint16_t*)sink_v;
  a.n_sink = n_sink;
  a.win_k = (const uint16_t*)win_k;
  a.win_v = (const uint16_t*)win_v;
  a.win_lens = win_cap > 0 ? win_lens : nullptr;
  a.win_cap = win_cap;
  a.out = out;
  a.partials = (float*)workspace;
  a.nsplit_of = nullptr;
  a.merge_pre = sp.max_split;
  a.nq = nq;
  a.q0 = q0;
  a.g_real = g_real > 0 ? g_real : L.G;
  a.k_new = app != nullptr ? (const uint16_t*)app->k : nullptr;
  a.v_new = app != nullptr ? (const uint16_t*)app->v : nullptr;
  a.pages_w = app != nullptr ? (uint8_t*)app->pages : nullptr;
  const dim3 mgrid0((unsigned)(num_seqs * L.Hkv * L.G));  // merge: one workgroup per query head
  if (tq_decode_block_format(L)) {  // whole-block streaming kernel (tq_decode_block.hip)
    if (a.rows_blocks > 0) {
      if (L.G <= 4) hipLaunchKernelGGL((tq_decode_rows_kernel<128, 4>), dim3(a.rows_blocks), dim3(kWG), 0, st, a);
      else hipLaunchKernelGGL((tq_decode_rows_kernel<128, 8>), dim3(a.rows_blocks), dim3(kWG), 0, st, a);
    }
    int32_t* nsplit = (int32_t*)((uint8_t*)workspace + partials_bytes(L, num_seqs, sp, n_sink, win_cap));
    const int e = tq_launch_decode_block(L, q, pages, block_tables, max_blocks, seq_lens, num_seqs, sp,
                                         n_sink, a.win_lens, win_cap, a.qscale, a.partials, nsplit,
                                         a.part_stride, nq, q0, a.g_real, stream, app);
    if (e != 0) return e;
    a.nsplit_of = nsplit;
    // the block kernel's aligned pieces: about 256 / num_seqs per sequence
    a.merge_pre = num_seqs > 0 ? (256 / num_seqs < sp.max_split ? 256 / num_seqs : sp.max_split) : 1;
    if (L.G <= 4) launch_merge<128, 4>(a, mgrid0, st);
    else launch_merge<128, 8>(a, mgrid0, st);
    return (int)hipGetLastError();
  }
  const long groups = (a.n_units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * L.Hkv));  // packed splits; launch_t adds the row chunks
  const dim3 mgrid((unsigned)(num_seqs * L.Hkv * L.G));
  if (L.D == 128) launch_k<128>(a, grid, mgrid, st);
  else launch_k<64>(a, grid, mgrid, st);
  return (int)hipGetLastError();
}
