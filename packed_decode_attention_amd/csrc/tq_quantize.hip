// Quantize-on-append and bit-exact dequantization kernels for gfx950.
//
// Quantize: turboquant-serve 0.1.2 "Architecture" (rotate, normalise, Lloyd-Max encode, bit-pack,
// store uint8); turboquant-pro 1.4.2 "How It Works" (per-vector flow: norm, normalise, rotate,
// quantise, pack, norm kept beside the bits); TorbuQuant docs "TQ4 page tensor" (slot layout).
// Dequantize: turboquant-serve 0.1.2 "Architecture" _decode (unpack, centroid lookup, restore
// magnitude, rotate back), with an exact fp64 Walsh-Hadamard transform so the fp32 result has a
// single fixed rounding chain.
//
// One row group of D/8 lanes per (token, kv head) row; lane j holds coordinates 8j..8j+7.

#include "tq_device.h"

namespace {
using namespace tqd;
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

}  // namespace

static float rsqrt_of(int D) { return (float)(1.0 / __builtin_sqrt((double)D)); }

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
