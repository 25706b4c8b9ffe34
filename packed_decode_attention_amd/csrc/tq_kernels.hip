// HIP kernels for gfx950 (CDNA4, wave64): quantize-on-append, fused paged decode attention over
// packed TQ pages, and bit-exact dequantization.
//
// Lane layout shared by all three kernels: a (token, kv head) row of D coordinates is owned by
// D/8 consecutive lanes ("row group"); lane j of the group holds coordinates 8j..8j+7.  With this
// layout the Walsh-Hadamard transform is three in-register butterfly stages (coordinate bits 0-2)
// followed by log2(D/8) cross-lane stages (coordinate bits 3..), and the packed codes of lane j are
// the `bits` bytes starting at byte bits*j of the region, so a row group reads its region with one
// coalesced access.
//
// Sources of the method: turboquant-serve 0.1.2 "Architecture" (rotate, normalise, Lloyd-Max
// encode, bit-pack; decode = unpack, centroid lookup, restore magnitude, rotate back); tq-kv
// "How It Works" [3] (randomized Hadamard transform) and "Custom CUDA Kernel Stack" (split-KV
// flash decode with online softmax, attention on compressed KV); TorbuQuant docs "TQ4 page tensor"
// (slot layout and addressing); turboquant-pro 1.4.2 "Fused CUDA decode" (split-K decode on codes).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace {

constexpr int kWG = 256;                    // threads per workgroup for every kernel here
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// 8 consecutive fp16 values (16-byte aligned) -> fp32.
__device__ __forceinline__ void load8_f16(const uint16_t* p, float x[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = half_bits_to_float(w[i] & 0xffffu);
    x[2 * i + 1] = half_bits_to_float(w[i] >> 16);
  }
}

// Sign bits of coordinates 8j..8j+7 (bit e set: s_{8j+e} = -1).
__device__ __forceinline__ uint32_t sign_byte(const TqSigns& s, int j) {
  return (s.w[(8 * j) >> 5] >> ((8 * j) & 31)) & 0xffu;
}

// The 8*bits code bits of lane j of a packed region (region start is 4-byte aligned).  The second
// dword read by the last lane is at most the region's norm, so it stays inside the slot.
__device__ __forceinline__ uint64_t lane_codes(const uint8_t* region, int bits, int j) {
  const int byte0 = bits * j;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(region) + (byte0 >> 2);
  const uint64_t both = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
  return both >> ((byte0 & 3) * 8);
}

// Walsh-Hadamard transform (Sylvester order) of the D values held by a row group, fp32.
template <int LPR, typename T>
__device__ __forceinline__ void wht_rowgroup(T x[8], int j) {
#pragma unroll
  for (int hb = 1; hb < 8; hb <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!(e & hb)) {
        const T a = x[e], b = x[e | hb];
        x[e] = a + b;
        x[e | hb] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    const bool upper = (j & m) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const T p = __shfl_xor(x[e], m, LPR);
      x[e] = upper ? p - x[e] : x[e] + p;
    }
  }
}

// =============================================================================================
// Quantize-on-append
// =============================================================================================
template <int D>
__device__ __forceinline__ void quantize_region(const uint16_t* __restrict__ src, int bits,
                                                int code_bytes, const float* s_t, uint32_t sbyte,
                                                int j, float rsqrt_d, uint8_t* __restrict__ dst) {
  constexpr int LPR = D / 8;
  float x[8];
  load8_f16(src + 8 * j, x);

  // Stored norm: exact fp32 squares, stride-halving tree (cross-lane levels h = D/2 .. 8, then
  // in-lane h = 4, 2, 1), correctly rounded square root (sqrtf; HIP's default device sqrtf is
  // correctly rounded, unlike the native instruction).  Contraction is off so every level is one
  // rounded fp32 add.
  const float n = [&] {
#pragma clang fp contract(off)
    float sq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[e] = x[e] * x[e];
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sq[e] = sq[e] + __shfl_xor(sq[e], m, LPR);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sq[e] = sq[e] + sq[e + 4];
    sq[0] = sq[0] + sq[2];
    sq[1] = sq[1] + sq[3];
    return sqrtf(sq[0] + sq[1]);
  }();

  // Rotation: sign flip, then the Walsh-Hadamard butterflies.
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((sbyte >> e) & 1u) x[e] = -x[e];
  wht_rowgroup<LPR>(x, j);

  // Nearest centroid = number of boundaries <= u (binary search over the sorted boundaries).
  const int levels = 1 << bits;
  uint64_t word = 0;
  if (n > 0.0f) {
    const float inv = rsqrt_d / n;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = x[e] * inv;
      int idx = 0;
      for (int s = levels >> 1; s >= 1; s >>= 1)
        if (s_t[idx + s - 1] <= u) idx += s;
      word |= (uint64_t)idx << (e * bits);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= (uint64_t)(levels >> 1) << (e * bits);
  }

  // Pack: lane j owns bytes [bits*j, bits*(j+1)) of the LSB-first bitstream.
  uint8_t* c = dst + bits * j;
  switch (bits) {
    case 2:
      *reinterpret_cast<uint16_t*>(c) = (uint16_t)word;
      break;
    case 4:
      *reinterpret_cast<uint32_t*>(c) = (uint32_t)word;
      break;
    case 8:
      reinterpret_cast<uint32_t*>(c)[0] = (uint32_t)word;
      reinterpret_cast<uint32_t*>(c)[1] = (uint32_t)(word >> 32);
      break;
    default:
      for (int i = 0; i < bits; ++i) c[i] = (uint8_t)(word >> (8 * i));
      break;
  }
  if (j == 0) *reinterpret_cast<float*>(dst + code_bytes) = n;
}

template <int D>
__global__ __launch_bounds__(kWG) void tq_quantize_kernel(TqLayer L, float rsqrt_d,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const int64_t* __restrict__ slot_mapping,
                                                          int64_t n_rows, uint8_t* __restrict__ pages) {
  constexpr int LPR = D / 8;
  constexpr int RPW = kWG / LPR;
  __shared__ float s_kt[256];
  __shared__ float s_vt[256];
  const int nkt = (1 << L.kb) - 1, nvt = (1 << L.vb) - 1;
  for (int i = threadIdx.x; i < nkt; i += kWG) s_kt[i] = L.kt[i];
  for (int i = threadIdx.x; i < nvt; i += kWG) s_vt[i] = L.vt[i];
  __syncthreads();

  const int j = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / LPR;
  if (row >= n_rows) return;
  const int64_t t = row / L.Hkv;
  const int h = (int)(row - t * L.Hkv);
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;
  uint8_t* dst = pages + (slot * L.Hkv + h) * (int64_t)L.stride;
  const uint32_t sb = sign_byte(L.signs, j);
  quantize_region<D>(k + row * D, L.kb, L.kcode_bytes, s_kt, sb, j, rsqrt_d, dst);
  quantize_region<D>(v + row * D, L.vb, L.vcode_bytes, s_vt, sb, j, rsqrt_d,
                     dst + L.kcode_bytes + 4);
  for (int i = L.slot_bytes + j; i < L.stride; i += LPR) dst[i] = 0;
}

// =============================================================================================
// Dequantize slots (bit-exact route: exact fp64 Walsh-Hadamard of the fp32 centroids)
// =============================================================================================
template <int D>
__device__ __forceinline__ void dequant_region(const uint8_t* __restrict__ region, int bits,
                                               int code_bytes, const float* s_c, uint32_t sbyte,
                                               int j, float rsqrt_d, float* __restrict__ out) {
  constexpr int LPR = D / 8;
  const uint64_t cw = lane_codes(region, bits, j);
  const uint32_t mask = (1u << bits) - 1u;
  double z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (double)s_c[(cw >> (e * bits)) & mask];
  wht_rowgroup<LPR>(z, j);  // exact: every partial sum fits in 53 bits
  const float n = *reinterpret_cast<const float*>(region + code_bytes);
  const float g = n * rsqrt_d;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float r = (float)z[e] * g;
    o[e] = ((sbyte >> e) & 1u) ? -r : r;
  }
  float4* o4 = reinterpret_cast<float4*>(out + 8 * j);
  o4[0] = make_float4(o[0], o[1], o[2], o[3]);
  o4[1] = make_float4(o[4], o[5], o[6], o[7]);
}

template <int D>
__global__ __launch_bounds__(kWG) void tq_dequant_kernel(TqLayer L, float rsqrt_d,
                                                         const uint8_t* __restrict__ pages,
                                                         const int64_t* __restrict__ slots,
                                                         int64_t n_rows, float* __restrict__ k_out,
                                                         float* __restrict__ v_out) {
  constexpr int LPR = D / 8;
  constexpr int RPW = kWG / LPR;
  __shared__ float s_kc[256];
  __shared__ float s_vc[256];
  for (int i = threadIdx.x; i < (1 << L.kb); i += kWG) s_kc[i] = L.kc[i];
  for (int i = threadIdx.x; i < (1 << L.vb); i += kWG) s_vc[i] = L.vc[i];
  __syncthreads();
  const int j = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / LPR;
  if (row >= n_rows) return;
  const int64_t i = row / L.Hkv;
  const int h = (int)(row - i * L.Hkv);
  const uint8_t* src = pages + (slots[i] * L.Hkv + h) * (int64_t)L.stride;
  const uint32_t sb = sign_byte(L.signs, j);
  dequant_region<D>(src, L.kb, L.kcode_bytes, s_kc, sb, j, rsqrt_d, k_out + row * D);
  dequant_region<D>(src + L.kcode_bytes + 4, L.vb, L.vcode_bytes, s_vc, sb, j, rsqrt_d,
                    v_out + row * D);
}

// =============================================================================================
// Fused paged decode attention (split-K, one workgroup per (sequence, kv head, split))
// =============================================================================================
// Workspace: [counters: B*Hkv uint32, padded to 256 B][partials: B*Hkv*max_split*G*(D+2) fp32]
// partial = (m, l, acc[D]) in the log2 domain and the rotated coordinate frame.

template <int D, int GMAX>
__global__ __launch_bounds__(kWG) void tq_decode_kernel(
    TqLayer L, float rsqrt_d, float qscale, float sink_scale, const uint16_t* __restrict__ q,
    const uint8_t* __restrict__ pages, const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ seq_lens, int chunk, int max_split,
    const uint16_t* __restrict__ sink_k, const uint16_t* __restrict__ sink_v, int n_sink,
    float* __restrict__ out, uint32_t* __restrict__ counters, float* __restrict__ partials) {
  constexpr int LPR = D / 8;
  constexpr int TPW = 64 / LPR;  // tokens in flight per wave
  constexpr int NW = kWG / 64;
  const int G = L.G;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int seq_len = seq_lens[b];
  const int ns = min(n_sink, seq_len);
  const int npage = seq_len - ns;
  const int nsplit = npage > 0 ? (npage + chunk - 1) / chunk : 1;
  if (split >= nsplit) return;

  __shared__ float s_kc[256];
  __shared__ float s_vc[256];
  __shared__ float s_part[NW][GMAX][D + 2];
  __shared__ int s_last;
  for (int i = threadIdx.x; i < (1 << L.kb); i += kWG) s_kc[i] = L.kc[i];
  for (int i = threadIdx.x; i < (1 << L.vb); i += kWG) s_vc[i] = L.vc[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % LPR;
  const int sub = lane / LPR;
  const uint32_t sb = sign_byte(L.signs, j);

  // Rotated, scaled query for the G heads of this kv head: qscale * H (s * q), qscale =
  // scale * log2(e) / sqrt(D), so scores come out in the log2 domain.
  float qr[GMAX][8];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      load8_f16(q + ((int64_t)b * L.Hq + h * G + g) * D + 8 * j, qr[g]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[g][e] = ((sb >> e) & 1u) ? -qr[g][e] : qr[g][e];
      wht_rowgroup<LPR>(qr[g], j);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[g][e] *= qscale;
    }
  }

  float m[GMAX], l[GMAX], acc[GMAX][8];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
  }

  const int p_begin = ns + split * chunk;
  const int p_end = min(ns + (split + 1) * chunk, seq_len);
  const int32_t* bt = block_tables + (int64_t)b * max_blocks;
  const uint32_t kmask = (1u << L.kb) - 1u, vmask = (1u << L.vb) - 1u;
  const int voff = L.kcode_bytes + 4;

  for (int p = p_begin + wave * TPW + sub; p < p_end; p += NW * TPW) {
    const int64_t slot = (int64_t)bt[p / L.bs] * L.bs + (p % L.bs);
    const uint8_t* base = pages + (slot * L.Hkv + h) * (int64_t)L.stride;
    const uint64_t kw = lane_codes(base, L.kb, j);
    const float kn = *reinterpret_cast<const float*>(base + L.kcode_bytes);
    const uint64_t vw = lane_codes(base + voff, L.vb, j);
    const float vn = *reinterpret_cast<const float*>(base + voff + L.vcode_bytes);
    float kf[8], vf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = s_kc[(kw >> (e * L.kb)) & kmask];
      vf[e] = s_vc[(vw >> (e * L.vb)) & vmask];
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g < G) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += qr[g][e] * kf[e];
#pragma unroll
        for (int msk = LPR / 2; msk >= 1; msk >>= 1) dot += __shfl_xor(dot, msk, LPR);
        const float s = kn * dot;
        const float m_new = fmaxf(m[g], s);
        const float sc = exp2f(m[g] - m_new);
        const float pw = exp2f(s - m_new);
        l[g] = l[g] * sc + pw;
        const float w = pw * vn;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = acc[g][e] * sc + w * vf[e];
        m[g] = m_new;
      }
    }
  }

  // Merge the TPW token streams of the wave (lanes with equal j hold the same coordinates).
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
#pragma unroll
      for (int msk = LPR; msk < 64; msk <<= 1) {
        const float mo = __shfl_xor(m[g], msk);
        const float lo = __shfl_xor(l[g], msk);
        const float M = fmaxf(m[g], mo);
        const float a = (m[g] == -INFINITY) ? 0.0f : exp2f(m[g] - M);
        const float ao = (mo == -INFINITY) ? 0.0f : exp2f(mo - M);
        l[g] = l[g] * a + lo * ao;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float o = __shfl_xor(acc[g][e], msk);
          acc[g][e] = acc[g][e] * a + o * ao;
        }
        m[g] = M;
      }
      if (sub == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_part[wave][g][2 + 8 * j + e] = acc[g][e];
        if (j == 0) {
          s_part[wave][g][0] = m[g];
          s_part[wave][g][1] = l[g];
        }
      }
    }
  }
  __syncthreads();

  // Merge the waves and publish this split's partial.
  const int64_t bh = (int64_t)b * L.Hkv + h;
  float* part = partials + (bh * max_split + split) * (int64_t)G * (D + 2);
  for (int i = threadIdx.x; i < G * (D + 2); i += kWG) {
    const int g = i / (D + 2), d = i % (D + 2);
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_part[w][g][0]);
    float r;
    if (d == 0) {
      r = M;
    } else {
      r = 0.0f;
      for (int w = 0; w < NW; ++w) {
        const float mw = s_part[w][g][0];
        const float a = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
        r += s_part[w][g][d] * a;
      }
    }
    part[i] = r;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&counters[bh], 1u);
    s_last = (prev == (uint32_t)(nsplit - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x == 0) counters[bh] = 0u;  // leave the counter zero for the next call

  // Last workgroup of this (sequence, kv head): merge splits, sinks, rotate back, normalise.
  float* s_acc = &s_part[0][0][0];                 // reuse: [G][D] rotated accumulators
  float* s_ml = &s_part[1][0][0];                  // [G] max, [G] sum
  float* s_sink = &s_part[2][0][0];                // [G][ns] sink scores (log2 domain)
  static_assert((NW - 2) * (D + 2) >= TQ_MAX_SINKS, "LDS too small for the sink scores");
  const int ns_eff = ns;                           // host guarantees n_sink <= TQ_MAX_SINKS
  if (seq_len == 0) {
    for (int i = threadIdx.x; i < G * D; i += kWG)
      out[((int64_t)b * L.Hq + h * G) * D + i] = 0.0f;
    return;
  }
  for (int i = threadIdx.x; i < G * ns_eff; i += kWG) {
    const int g = i / ns_eff, pp = i % ns_eff;
    const uint16_t* qv = q + ((int64_t)b * L.Hq + h * G + g) * D;
    const uint16_t* kv = sink_k + (((int64_t)b * n_sink + pp) * L.Hkv + h) * D;
    float dot = 0.0f;
    for (int d = 0; d < D; ++d) dot += half_bits_to_float(qv[d]) * half_bits_to_float(kv[d]);
    s_sink[g * ns_eff + pp] = dot * sink_scale;
  }
  __syncthreads();
  const float* pb = partials + bh * max_split * (int64_t)G * (D + 2);
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pb[(s * G + g) * (D + 2)]);
    for (int pp = 0; pp < ns_eff; ++pp) M = fmaxf(M, s_sink[g * ns_eff + pp]);
    float sum = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = pb[(s * G + g) * (D + 2)];
      if (ms != -INFINITY) sum += pb[(s * G + g) * (D + 2) + 1] * exp2f(ms - M);
    }
    for (int pp = 0; pp < ns_eff; ++pp) sum += exp2f(s_sink[g * ns_eff + pp] - M);
    s_ml[g] = M;
    s_ml[GMAX + g] = sum;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += kWG) {
    const int g = i / D, d = i % D;
    const float M = s_ml[g];
    float a = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = pb[(s * G + g) * (D + 2)];
      if (ms != -INFINITY) a += pb[(s * G + g) * (D + 2) + 2 + d] * exp2f(ms - M);
    }
    s_acc[g * D + d] = a;
  }
  __syncthreads();
  // Inverse rotation R^T a = D^(-1/2) diag(s) H a: Walsh-Hadamard butterflies in LDS.
  for (int hb = 1; hb < D; hb <<= 1) {
    for (int i = threadIdx.x; i < G * D / 2; i += kWG) {
      const int g = i / (D / 2), r = i % (D / 2);
      const int lo = (r / hb) * 2 * hb + (r % hb);
      const float a = s_acc[g * D + lo], c = s_acc[g * D + lo + hb];
      s_acc[g * D + lo] = a + c;
      s_acc[g * D + lo + hb] = a - c;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < G * D; i += kWG) {
    const int g = i / D, d = i % D;
    const bool neg = (L.signs.w[d >> 5] >> (d & 31)) & 1u;
    float o = s_acc[g * D + d] * rsqrt_d;
    if (neg) o = -o;
    const float M = s_ml[g];
    for (int pp = 0; pp < ns_eff; ++pp) {
      const float w = exp2f(s_sink[g * ns_eff + pp] - M);
      o += w * half_bits_to_float(sink_v[(((int64_t)b * n_sink + pp) * L.Hkv + h) * D + d]);
    }
    out[((int64_t)b * L.Hq + h * G + g) * D + d] = o / s_ml[GMAX + g];
  }
}

}  // namespace

// =============================================================================================
// Launchers
// =============================================================================================
static float rsqrt_of(int D) { return (float)(1.0 / __builtin_sqrt((double)D)); }

TqSplit tq_decode_split(const TqLayer& L, int num_seqs, int max_seq_len) {
  // Aim for enough workgroups to fill 256 CUs several times over; splits of >= 64 tokens.
  const long bh = (long)num_seqs * L.Hkv;
  const int target = 8192;
  int nsplit = (int)((target + bh - 1) / bh);
  const int max_tok = max_seq_len > 0 ? max_seq_len : 1;
  const int cap = (max_tok + 63) / 64;
  if (nsplit > cap) nsplit = cap;
  if (nsplit < 1) nsplit = 1;
  int chunk = (max_tok + nsplit - 1) / nsplit;
  chunk = ((chunk + 63) / 64) * 64;
  TqSplit sp;
  sp.chunk = chunk;
  sp.max_split = (max_tok + chunk - 1) / chunk;
  if (sp.max_split < 1) sp.max_split = 1;
  return sp;
}

size_t tq_decode_ws_bytes(const TqLayer& L, int num_seqs, const TqSplit& sp) {
  const size_t bh = (size_t)num_seqs * L.Hkv;
  const size_t counters = ((bh * 4 + 255) / 256) * 256;
  return counters + bh * (size_t)sp.max_split * L.G * (L.D + 2) * sizeof(float);
}

int tq_launch_quantize(const TqLayer& L, const void* k, const void* v, const int64_t* slot_mapping,
                       int64_t n_tok, void* pages, void* stream) {
  const int64_t rows = n_tok * L.Hkv;
  if (rows == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const int rpw = kWG / (L.D / 8);
  const dim3 grid((unsigned)((rows + rpw - 1) / rpw));
  if (L.D == 128)
    hipLaunchKernelGGL(tq_quantize_kernel<128>, grid, dim3(kWG), 0, st, L, rsqrt_of(128),
                       (const uint16_t*)k, (const uint16_t*)v, slot_mapping, rows, (uint8_t*)pages);
  else
    hipLaunchKernelGGL(tq_quantize_kernel<64>, grid, dim3(kWG), 0, st, L, rsqrt_of(64),
                       (const uint16_t*)k, (const uint16_t*)v, slot_mapping, rows, (uint8_t*)pages);
  return (int)hipGetLastError();
}

int tq_launch_dequant(const TqLayer& L, const void* pages, const int64_t* slots, int64_t n,
                      float* k_out, float* v_out, void* stream) {
  const int64_t rows = n * L.Hkv;
  if (rows == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const int rpw = kWG / (L.D / 8);
  const dim3 grid((unsigned)((rows + rpw - 1) / rpw));
  if (L.D == 128)
    hipLaunchKernelGGL(tq_dequant_kernel<128>, grid, dim3(kWG), 0, st, L, rsqrt_of(128),
                       (const uint8_t*)pages, slots, rows, k_out, v_out);
  else
    hipLaunchKernelGGL(tq_dequant_kernel<64>, grid, dim3(kWG), 0, st, L, rsqrt_of(64),
                       (const uint8_t*)pages, slots, rows, k_out, v_out);
  return (int)hipGetLastError();
}

template <int D, int GMAX>
static void launch_decode_t(const TqLayer& L, dim3 grid, hipStream_t st, float qscale,
                            const void* q, const void* pages, const int32_t* bt, int max_blocks,
                            const int32_t* seq_lens, const TqSplit& sp, const void* sk,
                            const void* sv, int n_sink, float* out, uint32_t* counters,
                            float* partials) {
  hipLaunchKernelGGL((tq_decode_kernel<D, GMAX>), grid, dim3(kWG), 0, st, L, rsqrt_of(D), qscale,
                     qscale * (float)(__builtin_sqrt((double)D)),
                     (const uint16_t*)q, (const uint8_t*)pages, bt, max_blocks, seq_lens, sp.chunk,
                     sp.max_split, (const uint16_t*)sk, (const uint16_t*)sv, n_sink, out, counters,
                     partials);
}

int tq_launch_decode(const TqLayer& L, const void* q, const void* pages, const int32_t* block_tables,
                     int max_blocks, const int32_t* seq_lens, int num_seqs, const TqSplit& sp,
                     const void* sink_k, const void* sink_v, int n_sink, float scale, float* out,
                     void* workspace, void* stream) {
  if (num_seqs == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const size_t bh = (size_t)num_seqs * L.Hkv;
  uint32_t* counters = (uint32_t*)workspace;
  float* partials = (float*)((char*)workspace + ((bh * 4 + 255) / 256) * 256);
  const dim3 grid(sp.max_split, L.Hkv, num_seqs);
  const float qscale = scale * kLog2e * rsqrt_of(L.D);
#define TQ_DECODE_CASE(DD, GG)                                                               \
  launch_decode_t<DD, GG>(L, grid, st, qscale, q, pages, block_tables, max_blocks, seq_lens, sp, \
                          sink_k, sink_v, n_sink, out, counters, partials)
  const int gb = L.G <= 1 ? 1 : L.G <= 2 ? 2 : L.G <= 4 ? 4 : 8;
  if (L.D == 128) {
    switch (gb) {
      case 1: TQ_DECODE_CASE(128, 1); break;
      case 2: TQ_DECODE_CASE(128, 2); break;
      case 4: TQ_DECODE_CASE(128, 4); break;
      default: TQ_DECODE_CASE(128, 8); break;
    }
  } else {
    switch (gb) {
      case 1: TQ_DECODE_CASE(64, 1); break;
      case 2: TQ_DECODE_CASE(64, 2); break;
      case 4: TQ_DECODE_CASE(64, 4); break;
      default: TQ_DECODE_CASE(64, 8); break;
    }
  }
#undef TQ_DECODE_CASE
  return (int)hipGetLastError();
}
