// Quantize-on-append and bit-exact dequantization kernels for gfx950.
//
// Quantize: turboquant-serve 0.1.2 "Architecture" (rotate, normalise, Lloyd-Max encode, bit-pack,
// store uint8); turboquant-pro 1.4.2 "How It Works" (per-vector flow: norm, normalise, rotate,
// quantise, pack, norm kept beside the bits); TorbuQuant docs "TQ4 page tensor" (slot layout).
// Dequantize: turboquant-serve 0.1.2 "Architecture" _decode (unpack, centroid lookup, restore
// magnitude, rotate back), with an exact fp64 Walsh-Hadamard transform so the fp32 result has a
// single fixed rounding chain.
//
// Quantize: D/16 lanes per (token, kv head) row, 16 coordinates each.  Dequantize: D/8 lanes per
// row, lane j holding coordinates 8j..8j+7.

#include "tq_device.h"

namespace {
using namespace tqd;
// =============================================================================================
// Quantize-on-append
//
// A row (one token and kv head, K or V) is held by P = D/16 lanes, 16 coordinates each.  Loads,
// decisions, packing and stores use the contiguous layout (lane j: coordinates 16j .. 16j + 15).
// The norm and the butterflies of coordinate bits >= log2(P) run in a transposed layout (lane j:
// coordinates j + P k, k = 0..15) reached through a per-wave LDS buffer: there the first levels of
// the norm tree (pairs i, i + D/2, then D/4, ...) and those butterflies are in-lane, and only the
// last log2(P) norm levels cross lanes (DPP).  A second pass through the buffer returns to the
// contiguous layout for the low-bit butterflies.
//
// Decisions: idx = #{j : t_j <= u}.  With S a power of two no smaller than 1 / (smallest gap between
// boundaries), the bucket floor(u S) holds at most one boundary; a table gives per bucket the
// number of boundaries below it and the next boundary times S, so idx = base + (u S >= S t).  u S
// scales u exactly, so the decision is the comparison of u with the fp32 boundaries.  A codebook
// whose boundaries are closer than the table allows falls back to a binary search.
// =============================================================================================
constexpr int kQTabSmall = 130;   // bucket-table entries for codes of up to 4 bits (S <= 64)
constexpr int kQTabLarge = 2050;  // for 8-bit codes (S <= 1024)
constexpr int kQNoTable = -100;   // log2 S marker: binary search

__host__ __device__ constexpr int qtab_entries(int bits) { return bits <= 4 ? kQTabSmall : kQTabLarge; }

// 16 contiguous fp16 of lane j (signs flipped), transposed through the row's LDS buffer, as fp32
// coordinates j + P k of the row, k = 0..15.
template <int P>
__device__ __forceinline__ void to_transposed(const uint32_t (&raw)[8], uint32_t* xr, int j, float (&y)[16]) {
  // coordinate c = 16 j + m goes to transposed row c % P at column c / P (fp16 positions)
  if constexpr (P == 8) {
#pragma unroll
    for (int m = 0; m < 8; ++m)  // (m, m + 8): one dword of row m, column pair j
      xr[m * 8 + j] = __builtin_amdgcn_perm(raw[4 + m / 2], raw[m / 2], (m & 1) ? 0x07060302u : 0x05040100u);
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {  // (m, m + 4), (m + 8, m + 12): two dwords of row m, columns 4j..
      const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t w0 = __builtin_amdgcn_perm(raw[m / 2 + 2], raw[m / 2], sel);
      const uint32_t w1 = __builtin_amdgcn_perm(raw[m / 2 + 6], raw[m / 2 + 4], sel);
      *reinterpret_cast<uint2*>(xr + m * 8 + 2 * j) = make_uint2(w0, w1);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const uint4 a = reinterpret_cast<const uint4*>(xr + 8 * j)[0];
  const uint4 b = reinterpret_cast<const uint4*>(xr + 8 * j)[1];
  const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    y[2 * q] = half_bits_to_float(d[q] & 0xffffu);
    y[2 * q + 1] = half_bits_to_float(d[q] >> 16);
  }
}

// One region (K or V) of P lanes' row: norm, rotation, decisions, packing, store.
template <int D>
__device__ __forceinline__ void quantize_row(const uint16_t* __restrict__ src, bool load,
                                             const uint32_t (&smask)[8], uint32_t* xr, int j, int bits,
                                             int code_bytes, const float* s_t, const uint2* tab, int sh,
                                             float rsqrt_d, uint8_t* __restrict__ dst, bool store) {
  constexpr int P = D / 16;
  uint32_t raw[8];
  if (load) {
    const uint4 a = reinterpret_cast<const uint4*>(src + 16 * j)[0];
    const uint4 b = reinterpret_cast<const uint4*>(src + 16 * j)[1];
    raw[0] = a.x; raw[1] = a.y; raw[2] = a.z; raw[3] = a.w;
    raw[4] = b.x; raw[5] = b.y; raw[6] = b.z; raw[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = 0;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) raw[i] ^= smask[i];  // sign flip on the fp16 sign bits
  float y[16];
  to_transposed<P>(raw, xr, j, y);

  // Stored norm: exact fp32 squares, stride-halving tree (pairs i, i + D/2, then D/4, ...: the
  // first four levels are k, k + 8 / 4 / 2 / 1 in-lane, the rest lane j, j + P/2 ...), correctly
  // rounded square root.  Contraction off: every level is one rounded fp32 add.
  const float n = [&] {
#pragma clang fp contract(off)
    float sq[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sq[e] = y[e] * y[e];
#pragma unroll
    for (int hf = 8; hf >= 1; hf >>= 1) {
#pragma unroll
      for (int e = 0; e < hf; ++e) sq[e] = sq[e] + sq[e + hf];
    }
    float s = sq[0];
    if constexpr (P == 8) s = s + dpp_xor<4>(s);
    s = s + dpp_xor<2>(s);
    s = s + dpp_xor<1>(s);
    return sqrtf(s);
  }();

  // Butterflies of coordinate bits log2(P) .. log2(D) - 1 (k bits), in-lane.
#pragma unroll
  for (int hb = 1; hb < 16; hb <<= 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (!(e & hb)) {
        const float a0 = y[e], b0 = y[e | hb];
        y[e] = a0 + b0;
        y[e | hb] = a0 - b0;
      }
    }
  }
  // Back to the contiguous layout through the same buffer.
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int e = 0; e < 16; ++e) xr[j + P * e] = __float_as_uint(y[e]);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  float z[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = reinterpret_cast<const uint4*>(xr + 16 * j)[i];
    z[4 * i] = __uint_as_float(w.x);
    z[4 * i + 1] = __uint_as_float(w.y);
    z[4 * i + 2] = __uint_as_float(w.z);
    z[4 * i + 3] = __uint_as_float(w.w);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // buffer free for the next row
  // Butterflies of coordinate bits 0 .. log2(P) - 1, in-lane.
#pragma unroll
  for (int hb = 1; hb < P; hb <<= 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (!(e & hb)) {
        const float a0 = z[e], b0 = z[e | hb];
        z[e] = a0 + b0;
        z[e | hb] = a0 - b0;
      }
    }
  }

  // Decisions: u = z / (sqrt(D) n); all indices 2^bits / 2 for a zero row (u = 0).
  const int levels = 1 << bits;
  uint32_t code[16];
  if (sh != kQNoTable) {
    const float inv = n > 0.0f ? ldexpf(rsqrt_d / n, sh) : 0.0f;  // S / (sqrt(D) n)
    const int off = (1 << sh) + 1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float us = z[e] * inv;
      const uint2 ent = tab[(int)floorf(us) + off];
      code[e] = ent.y + (us >= __uint_as_float(ent.x) ? 1u : 0u);
    }
  } else {
    const float inv = n > 0.0f ? rsqrt_d / n : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float u = z[e] * inv;
      int idx = 0;
      for (int st = levels >> 1; st >= 1; st >>= 1)
        if (s_t[idx + st - 1] <= u) idx += st;
      code[e] = (uint32_t)idx;
    }
  }

  // Pack: lane j owns bytes [2 bits j, 2 bits (j + 1)) of the LSB-first bitstream.
  if (store) {
    uint8_t* c = dst + 2 * bits * j;
    if (bits == 8) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = code[4 * i] | (code[4 * i + 1] << 8) | (code[4 * i + 2] << 16) | (code[4 * i + 3] << 24);
      *reinterpret_cast<uint4*>(c) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if (bits == 4) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        w0 |= code[e] << (4 * e);
        w1 |= code[e + 8] << (4 * e);
      }
      *reinterpret_cast<uint2*>(c) = make_uint2(w0, w1);
    } else if (bits == 2) {
      uint32_t w0 = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) w0 |= code[e] << (2 * e);
      *reinterpret_cast<uint32_t*>(c) = w0;
    } else {  // 3 bits: 48 bits at byte 6 j (2-byte aligned)
      uint64_t w = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) w |= (uint64_t)code[e] << (3 * e);
      uint16_t* c16 = reinterpret_cast<uint16_t*>(c);
      c16[0] = (uint16_t)w;
      c16[1] = (uint16_t)(w >> 16);
      c16[2] = (uint16_t)(w >> 32);
    }
    if (j == 0) *reinterpret_cast<float*>(dst + code_bytes) = n;
  }
}

// Bucket table of one codebook (see above): entries for buckets k = -(S + 1) .. S, entry
// {S t_base as bits, base} with base = #{t < k / S}.
__device__ __forceinline__ void build_qtab(const float* s_t, int nb, int sh, uint2* tab, int tid) {
  const int S = 1 << sh;
  for (int i = tid; i < 2 * S + 2; i += kWG) {
    const float edge = ldexpf((float)(i - (S + 1)), -sh);
    int lo = 0, hi = nb;  // first boundary >= edge
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_t[mid] < edge) lo = mid + 1;
      else hi = mid;
    }
    const float next = lo < nb ? ldexpf(s_t[lo], sh) : 3.0e38f;
    tab[i] = make_uint2(__float_as_uint(next), (uint32_t)lo);
  }
}

template <int D>
__global__ __launch_bounds__(kWG) void tq_quantize_kernel(TqLayer L, float rsqrt_d,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const int64_t* __restrict__ slot_mapping,
                                                          int64_t n_rows, uint8_t* __restrict__ pages) {
  constexpr int P = D / 16;    // lanes per row
  constexpr int RPW = 64 / P;  // rows per wave per step
  constexpr int XROW = D + 8;  // dwords per row of the transpose buffer (padded)
  constexpr int kNWQ = kWG / 64;
  __shared__ float s_t[2][256];
  __shared__ int s_sh[2];
  __shared__ __align__(16) uint32_t s_x[kNWQ][RPW * XROW];
  extern __shared__ uint2 s_tab[];  // K table (qtab_entries(kb)), then V table

  const int tid = threadIdx.x;
  const int nbk = (1 << L.kb) - 1, nbv = (1 << L.vb) - 1;
  for (int i = tid; i < nbk; i += kWG) s_t[0][i] = L.kt[i];
  for (int i = tid; i < nbv; i += kWG) s_t[1][i] = L.vt[i];
  __syncthreads();
  if (tid < 2) {  // table resolution per codebook: S = 2^sh >= 1 / (smallest gap)
    const int nb = tid == 0 ? nbk : nbv;
    float g = 2.0f;
    for (int i = 0; i + 1 < nb; ++i) g = fminf(g, s_t[tid][i + 1] - s_t[tid][i]);
    int sh = g > 0.0f ? -ilogbf(g) : kQNoTable;  // bucket width 2^-sh <= g
    if (sh < 0) sh = 0;
    if (g <= 0.0f || 2 * (1 << min(sh, 20)) + 2 > qtab_entries(tid == 0 ? L.kb : L.vb)) sh = kQNoTable;
    s_sh[tid] = sh;
  }
  __syncthreads();
  uint2* tabk = s_tab;
  uint2* tabv = s_tab + qtab_entries(L.kb);
  if (s_sh[0] != kQNoTable) build_qtab(s_t[0], nbk, s_sh[0], tabk, tid);
  if (s_sh[1] != kQNoTable) build_qtab(s_t[1], nbv, s_sh[1], tabv, tid);
  __syncthreads();
  const int shk = s_sh[0], shv = s_sh[1];

  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane % P, rr = lane / P;
  uint32_t* xr = &s_x[wave][rr * XROW];
  // fp16 sign masks of coordinates 16 j .. 16 j + 15 (bit 15 / 31 of dword i for 2i / 2i + 1)
  uint32_t smask[8];
  {
    const uint32_t sm = (L.signs.w[j >> 1] >> (16 * (j & 1))) & 0xffffu;
#pragma unroll
    for (int i = 0; i < 8; ++i) smask[i] = (((sm >> (2 * i)) & 1u) << 15) | (((sm >> (2 * i + 1)) & 1u) << 31);
  }
  const int64_t step = (int64_t)gridDim.x * kNWQ * RPW;
  for (int64_t r0 = ((int64_t)blockIdx.x * kNWQ + wave) * RPW; r0 < n_rows; r0 += step) {
    const int64_t row = r0 + rr;
    const bool in = row < n_rows;
    const int64_t t = in ? row / L.Hkv : 0;
    const int h = (int)(row - t * L.Hkv);
    const int64_t slot = in ? slot_mapping[t] : -1;
    const bool live = slot >= 0;
    uint8_t* dst = pages + (live ? (slot * L.Hkv + h) * (int64_t)L.stride : 0);
    quantize_row<D>(k + row * D, in, smask, xr, j, L.kb, L.kcode_bytes, s_t[0], tabk, shk, rsqrt_d, dst, live);
    quantize_row<D>(v + row * D, in, smask, xr, j, L.vb, L.vcode_bytes, s_t[1], tabv, shv, rsqrt_d,
                    dst + L.kcode_bytes + 4, live);
    if (live)
      for (int i = L.slot_bytes + j; i < L.stride; i += P) dst[i] = 0;
  }
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

}  // namespace

static float rsqrt_of(int D) { return (float)(1.0 / __builtin_sqrt((double)D)); }

int tq_launch_quantize(const TqLayer& L, const void* k, const void* v, const int64_t* slot_mapping,
                       int64_t n_tok, void* pages, void* stream) {
  const int64_t rows = n_tok * L.Hkv;
  if (rows == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const int64_t rows_per_wg = (kWG / 64) * (64 / (L.D / 16));
  const int64_t wgs = (rows + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)(wgs < 2048 ? wgs : 2048));  // workgroups loop over row groups
  const size_t tab_bytes = (size_t)(qtab_entries(L.kb) + qtab_entries(L.vb)) * sizeof(uint2);
  if (L.D == 128)
    hipLaunchKernelGGL(tq_quantize_kernel<128>, grid, dim3(kWG), tab_bytes, st, L, rsqrt_of(128),
                       (const uint16_t*)k, (const uint16_t*)v, slot_mapping, rows, (uint8_t*)pages);
  else
    hipLaunchKernelGGL(tq_quantize_kernel<64>, grid, dim3(kWG), tab_bytes, st, L, rsqrt_of(64),
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
