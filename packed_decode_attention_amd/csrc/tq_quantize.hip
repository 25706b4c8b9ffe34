// Quantize-on-append and bit-exact dequantization kernels for gfx950.
//
// Quantize: turboquant-serve 0.1.2 "Architecture" (rotate, normalise, Lloyd-Max encode, bit-pack,
// store uint8); turboquant-pro 1.4.2 "How It Works" (per-vector flow: norm, normalise, rotate,
// quantise, pack, norm kept beside the bits); tq-kv "How It Works" (randomised Hadamard
// rotation); TorbuQuant docs "TQ4 page tensor" (slot layout).
// Dequantize: turboquant-serve 0.1.2 "Architecture" _decode (unpack, centroid lookup, restore
// magnitude, rotate back), with an exact fp64 Walsh-Hadamard transform so the fp32 result has a
// single fixed rounding chain.

#include <type_traits>

#include "tq_quant_device.h"

namespace {
using namespace tqd;
using namespace tqq;

// Destination of the stores of rows that have no slot (past the end of the input, or a negative
// slot id): every lane stores on every tile, so each tile issues a fixed number of stores.
__device__ __align__(16) uint8_t tq_quant_discard[4096];

// Stores a region issues per tile (two for 8-bit codes, one otherwise, plus the norm (and mean)),
// and the
// s_waitcnt immediate that waits for everything issued before the last n vector memory operations
// (gfx9 encoding: vmcnt in bits 3..0 and 15..14; expcnt and lgkmcnt at their maxima).
constexpr int region_stores(int bits) { return (bits == 8 ? 2 : 1) + 1; }
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xf00; }

// Four waves per SIMD (128 VGPRs): the occupancy that keeps a tile of loads in flight per wave;
// without the attribute the fallback loop's pressure lowers it for the whole kernel.
// 4 waves per SIMD (at most 128 VGPRs); the mean-removal format, which also holds the centred row
// as fp16 high and low parts, gets 3 (168 VGPRs) so that nothing spills into the tile loop.
template <int D, int KB, int VB, bool NC, bool MEAN>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(MEAN ? 3 : 4))) void tq_quantize_kernel(
    TqLayer L, float rsqrt_d, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, int64_t n_rows, uint8_t* __restrict__ pages) {
  constexpr int NB = D / 32;
  constexpr int kNWQ = kWG / 64;
  __shared__ float s_t[2][256];
  __shared__ int s_sh[2];
  __shared__ float s_gap[kNWQ][2];
  __shared__ float s_c[2][NC ? 256 : 1];  // centroids (norm-correction format)
  // per wave: K blocks, V blocks, then the low and high dwords of the rows' slot ids
  __shared__ __align__(16) uint8_t s_stage[kNWQ][2 * NB * 1024 + 512];
  extern __shared__ uint2 s_tab[];  // K table (qtab_entries(kb)), then V table

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;

  // Each wave stages its next tile in its own LDS buffer (global_load_lds: lane l's 16 bytes of
  // block b land at b * 1024 + 16 l, the same lane reads them back; the slot id of lane l's row
  // lands as two dwords) while it works on the current one from registers.  All vector memory
  // operations share one in-order counter: the next tile's loads are issued before the current
  // tile's stores, and the wait at the top of an iteration lets exactly those stores stay in
  // flight.  The first tile's loads go out before the codebook is read, so that their latency
  // overlaps the table build (a small append is that one tile).
  uint8_t* stage = s_stage[wave];
  const int64_t n_tiles = (n_rows + 15) / 16;
  const int64_t tstep = (int64_t)gridDim.x * kNWQ;
  constexpr int kStores = region_stores(KB) + region_stores(VB);
  auto issue = [&](int64_t T) {
    const int64_t row = T * 16 + c;
    const int64_t rr = row < n_rows ? row : n_rows - 1;  // rows past the end load the last row
    const uint16_t* sk = k + rr * D + 8 * g;
    const uint16_t* sv = v + rr * D + 8 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      __builtin_amdgcn_global_load_lds(sk + 32 * b, stage + b * 1024, 16, 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b)
      __builtin_amdgcn_global_load_lds(sv + 32 * b, stage + (NB + b) * 1024, 16, 0, 0);
    const uint32_t* sl = reinterpret_cast<const uint32_t*>(slot_mapping + rr / L.Hkv);
    __builtin_amdgcn_global_load_lds(sl, stage + 2 * NB * 1024, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(sl + 1, stage + 2 * NB * 1024 + 256, 4, 0, 0);
  };
  const int64_t T0 = (int64_t)blockIdx.x * kNWQ + wave;
  if (T0 < n_tiles) issue(T0);

  // The codebooks (at most one boundary and one centroid per thread), then, while they load, the
  // Hadamard operands, which depend on no load.
  constexpr int nbk = (1 << KB) - 1, nbv = (1 << VB) - 1;
  static_assert(nbk < kWG && nbv < kWG, "one boundary gap per thread");
  const float tk = L.kt[min(tid, nbk - 1)];
  const float tv = L.vt[min(tid, nbv - 1)];
  float ck = 0.0f, cv = 0.0f;
  if constexpr (NC) {
    ck = L.kc[min(tid, nbk)];
    cv = L.vc[min(tid, nbv)];
  }
  // Hadamard A operands, computed while the codebook loads are in flight (the empty asm keeps
  // the compiler from sinking them past the table build)
  uint4 A[NB][2];
  hadamard_operands<NB>(L.signs, lane, A);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      asm volatile("" : "+v"(A[b][t].x), "+v"(A[b][t].y), "+v"(A[b][t].z), "+v"(A[b][t].w));
  if (tid < nbk) s_t[0][tid] = tk;
  if (tid < nbv) s_t[1][tid] = tv;
  if constexpr (NC) {
    if (tid <= nbk) s_c[0][tid] = ck;
    if (tid <= nbv) s_c[1][tid] = cv;
  }
  __syncthreads();
  {  // smallest gap between consecutive boundaries, one gap per thread (at most 254 of them)
    float gk = tid + 1 < nbk ? s_t[0][tid + 1] - s_t[0][tid] : 2.0f;
    float gv = tid + 1 < nbv ? s_t[1][tid + 1] - s_t[1][tid] : 2.0f;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      gk = fminf(gk, __shfl_xor(gk, m));
      gv = fminf(gv, __shfl_xor(gv, m));
    }
    if ((tid & 63) == 0) {
      s_gap[tid >> 6][0] = gk;
      s_gap[tid >> 6][1] = gv;
    }
  }
  __syncthreads();
  if (tid < 2) {  // table resolution per codebook: S = 2^sh >= 1 / (smallest gap)
    float gap = 2.0f;
    for (int w = 0; w < kNWQ; ++w) gap = fminf(gap, s_gap[w][tid]);
    s_sh[tid] = qtab_shift(gap, tid == 0 ? KB : VB);
  }
  __syncthreads();
  const int shk = s_sh[0], shv = s_sh[1];
  uint2* tabk = s_tab;
  uint2* tabv = s_tab + qtab_entries(KB);
  build_qtabs<KB, VB>(s_t, shk, shv, tabk, tabv, tid);
  __syncthreads();
  float zero;  // an addend of 0 the compiler cannot fold, so a lone square stays one v_fma_mix
  asm("v_mov_b32 %0, 0" : "=v"(zero));

  // Two complete tile loops, one per decision method (a codebook too fine for its table sends
  // both regions to the binary search), so neither loop carries the other's registers.
  auto tile_loop = [&](auto use_table) {
    constexpr bool kTable = decltype(use_table)::value;
    int64_t T = T0;  // its loads are in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    for (; T < n_tiles; T += tstep) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kStores));  // all but the previous tile's stores
      uint4 xk[NB], xv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) xk[b] = reinterpret_cast<const uint4*>(stage + b * 1024)[lane];
#pragma unroll
      for (int b = 0; b < NB; ++b) xv[b] = reinterpret_cast<const uint4*>(stage + (NB + b) * 1024)[lane];
      const uint32_t slo = reinterpret_cast<const uint32_t*>(stage + 2 * NB * 1024)[lane];
      const uint32_t shi = reinterpret_cast<const uint32_t*>(stage + 2 * NB * 1024 + 256)[lane];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): buffer read out before it is refilled
      const int64_t row = T * 16 + c;
      const int64_t slot = (int64_t)(((uint64_t)shi << 32) | slo);
      const bool live = row < n_rows && slot >= 0;
      const int64_t tok = row / L.Hkv;
      const int h = (int)(row - tok * L.Hkv);
      uint8_t* dst = live ? pages + (slot * L.Hkv + h) * (int64_t)L.stride : tq_quant_discard;
      for (int i = L.slot_bytes + g; i < L.stride; i += 4) dst[i] = 0;  // padding, before the loads
      if (T + tstep < n_tiles) issue(T + tstep);

      if constexpr (NC || MEAN) {  // each region stored as it is done
        quantize_region<D, KB, kTable, NC, MEAN>(xk, A, zero, g, L.kcode_bytes, s_t[0], tabk, shk,
                                                 s_c[0], rsqrt_d, dst);
        quantize_region<D, VB, kTable, NC, MEAN>(xv, A, zero, g, L.vcode_bytes, s_t[1], tabv, shv,
                                                 s_c[1], rsqrt_d, dst + L.kreg);
      } else {
        // Both regions first, then all of the tile's stores back to back: a row's K and V bytes
        // share cache lines, which then fill completely before the L2 can write them back (K
        // stored while V was still being computed left lines to be written back in two parts).
        const RegionBits<KB> rk = quantize_region_bits<D, KB, kTable, NC, MEAN>(xk, A, zero, s_t[0], tabk,
                                                                               shk, s_c[0], rsqrt_d);
        const RegionBits<VB> rv = quantize_region_bits<D, VB, kTable, NC, MEAN>(xv, A, zero, s_t[1], tabv,
                                                                               shv, s_c[1], rsqrt_d);
        store_region<D, KB, MEAN>(rk, g, L.kcode_bytes, dst);
        store_region<D, VB, MEAN>(rv, g, L.vcode_bytes, dst + L.kreg);
      }
    }
  };
  if (shk != kQNoTable && shv != kQNoTable) tile_loop(std::true_type{});
  else tile_loop(std::false_type{});
}

// =============================================================================================
// Dequantize slots (bit-exact route: exact fp64 Walsh-Hadamard of the fp32 centroids)
// =============================================================================================
// 1-bit QJL key residual (tq-kv, "How It Works", step [5]; the QJL estimator of the TurboQuant
// paper): sqrt(pi/2) / D times gamma times S^T z, in the rotated frame.
constexpr double kQjlKappa = 1.2533141373155002512;  // sqrt(pi / 2)

template <int D>
__device__ __forceinline__ void dequant_region(const uint8_t* __restrict__ region, int bits,
                                               int code_bytes, const float* s_c, uint32_t sbyte,
                                               int j, float rsqrt_d, int mean, float* __restrict__ out,
                                               int qjl_off = -1, uint32_t sbyte2 = 0) {
#pragma clang fp contract(off)
  constexpr int LPR = D / 8;
  const uint64_t cw = lane_codes(region, bits, j);
  const uint32_t mask = (1u << bits) - 1u;
  double z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (double)s_c[(cw >> (e * bits)) & mask];
  wht_rowgroup<LPR>(z, j);  // exact: every partial sum fits in 53 bits
  const float n = *reinterpret_cast<const float*>(region + code_bytes);
  const float g = n * rsqrt_d;
  // QJL key format: t = H diag(sigma2) H z, exact in fp64 (integers below D^2); its weight
  // sqrt(pi/2) / D * gamma * D^(-1/2) makes R^T of the sketched residual.
  double t[8];
  float gq = 0.0f;
  if (qjl_off >= 0) {
    const uint32_t zb = region[qjl_off + j];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = ((zb >> e) & 1u) ? 1.0 : -1.0;
    wht_rowgroup<LPR>(t, j);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((sbyte2 >> e) & 1u) t[e] = -t[e];
    wht_rowgroup<LPR>(t, j);
    const float gamma = *reinterpret_cast<const float*>(region + qjl_off + D / 8);
    gq = (float)(kQjlKappa / D * (double)gamma * (double)rsqrt_d);
  }
  float o[8];
  const float mu = mean ? *reinterpret_cast<const float*>(region + code_bytes + 4) : 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float r = (float)z[e] * g;
    if (qjl_off >= 0) r = r + (float)t[e] * gq;
    o[e] = ((sbyte >> e) & 1u) ? -r : r;
    if (mean) o[e] = o[e] + mu;  // mean-removal format: fp32(x_hat + mu)
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
  dequant_region<D>(src, L.kb, L.kcode_bytes, s_kc, sb, j, rsqrt_d, L.mean, k_out + row * D,
                    L.qjl ? L.kqjl : -1, sign_byte(L.signs2, j));
  dequant_region<D>(src + L.kreg, L.vb, L.vcode_bytes, s_vc, sb, j, rsqrt_d, L.mean,
                    v_out + row * D);
}

// QJL key format: the residual sketch of the keys tq_quantize_kernel has just written (same
// stream, so its codes, norm and mean are in place).  D/8 lanes per row, 8 coordinates each, in
// fp64 so the stored bytes are reproducible: d = x - mu and H (s * d) are exact in fp64 (fp16
// inputs, an fp32 mean); v = H (s * d) / sqrt(D) = R (x - mu 1), r = v - n_s c[idx] (n_s c is
// exact), gamma = fp32(||r||), then S r = H (sigma2 * r) and b = [(S r)_i >= 0], one byte per
// lane.  Only the fp64 roundings of v, r and S r (about 1e-15 of gamma) separate these from an
// exact computation.
template <int P>
__device__ __forceinline__ double group_sum_f64(double x) {
#pragma unroll
  for (int m = 1; m < P; m <<= 1) x += __shfl_xor(x, m, P);
  return x;
}

template <int D>
__global__ __launch_bounds__(kWG) void tq_qjl_kernel(TqLayer L, double rsqrt_d,
                                                     const uint16_t* __restrict__ k,
                                                     const int64_t* __restrict__ slot_mapping,
                                                     int64_t n_rows, uint8_t* __restrict__ pages) {
  constexpr int P = D / 8;
  constexpr int RPW = kWG / P;
  __shared__ float s_kc[256];
  for (int i = threadIdx.x; i < (1 << L.kb); i += kWG) s_kc[i] = L.kc[i];
  __syncthreads();
  const int j = threadIdx.x % P;
  // grid-stride over groups of RPW rows; a row group skips a row as a whole, so the cross-lane
  // steps stay inside active groups
  for (int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / P; row < n_rows;
       row += (int64_t)gridDim.x * RPW) {
    const int64_t t = row / L.Hkv;
    const int h = (int)(row - t * L.Hkv);
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    uint8_t* dst = pages + (slot * L.Hkv + h) * (int64_t)L.stride;
    float xf[8];
    load8_f16(k + row * D + 8 * j, xf);
    const double mu = L.mean ? (double)*reinterpret_cast<const float*>(dst + L.kcode_bytes + 4) : 0.0;
    const uint32_t sb = sign_byte(L.signs, j);
    double x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double d = (double)xf[e] - mu;
      x[e] = ((sb >> e) & 1u) ? -d : d;
    }
    wht_rowgroup<P>(x, j);
    const double ns = (double)*reinterpret_cast<const float*>(dst + L.kcode_bytes);
    const uint64_t cw = lane_codes(dst, L.kb, j);
    const uint32_t mask = (1u << L.kb) - 1u;
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double r = x[e] * rsqrt_d - ns * (double)s_kc[(cw >> (e * L.kb)) & mask];
      x[e] = r;
      ss += r * r;
    }
    const float gamma = (float)sqrt(group_sum_f64<P>(ss));
    const uint32_t sb2 = sign_byte(L.signs2, j);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((sb2 >> e) & 1u) x[e] = -x[e];
    wht_rowgroup<P>(x, j);
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) bits |= (x[e] >= 0.0 ? 1u : 0u) << e;
    dst[L.kqjl + j] = (uint8_t)bits;
    if (j == 0) *reinterpret_cast<float*>(dst + L.kqjl + D / 8) = gamma;
  }
}

}  // namespace

static float rsqrt_of(int D) { return (float)(1.0 / __builtin_sqrt((double)D)); }

template <int D, int KB, int VB>
static void launch_quantize(const TqLayer& L, dim3 grid, size_t lds, hipStream_t st, const void* k,
                            const void* v, const int64_t* slot_mapping, int64_t rows, void* pages) {
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kWG), lds, st, L, rsqrt_of(D), (const uint16_t*)k,
                       (const uint16_t*)v, slot_mapping, rows, (uint8_t*)pages);
  };
  if (L.norm_corr && L.mean) go(tq_quantize_kernel<D, KB, VB, true, true>);
  else if (L.norm_corr) go(tq_quantize_kernel<D, KB, VB, true, false>);
  else if (L.mean) go(tq_quantize_kernel<D, KB, VB, false, true>);
  else go(tq_quantize_kernel<D, KB, VB, false, false>);
}

template <int D, int KB>
static bool dispatch_vb(const TqLayer& L, dim3 grid, size_t lds, hipStream_t st, const void* k,
                        const void* v, const int64_t* sm, int64_t rows, void* pages) {
  switch (L.vb) {
    case 2: launch_quantize<D, KB, 2>(L, grid, lds, st, k, v, sm, rows, pages); return true;
    case 3: launch_quantize<D, KB, 3>(L, grid, lds, st, k, v, sm, rows, pages); return true;
    case 4: launch_quantize<D, KB, 4>(L, grid, lds, st, k, v, sm, rows, pages); return true;
    case 8: launch_quantize<D, KB, 8>(L, grid, lds, st, k, v, sm, rows, pages); return true;
  }
  return false;
}

template <int D>
static bool dispatch_kb(const TqLayer& L, dim3 grid, size_t lds, hipStream_t st, const void* k,
                        const void* v, const int64_t* sm, int64_t rows, void* pages) {
  switch (L.kb) {
    case 2: return dispatch_vb<D, 2>(L, grid, lds, st, k, v, sm, rows, pages);
    case 3: return dispatch_vb<D, 3>(L, grid, lds, st, k, v, sm, rows, pages);
    case 4: return dispatch_vb<D, 4>(L, grid, lds, st, k, v, sm, rows, pages);
    case 8: return dispatch_vb<D, 8>(L, grid, lds, st, k, v, sm, rows, pages);
  }
  return false;
}

int tq_launch_quantize(const TqLayer& L, const void* k, const void* v, const int64_t* slot_mapping,
                       int64_t n_tok, void* pages, void* stream) {
  const int64_t rows = n_tok * L.Hkv;
  if (rows == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const int64_t rows_per_wg = (kWG / 64) * 16;  // one 16-row tile per wave
  const int64_t wgs = (rows + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid((unsigned)(wgs < 2048 ? wgs : 2048));  // workgroups loop over tiles
  const size_t tab_bytes = (size_t)(qtab_entries(L.kb) + qtab_entries(L.vb)) * sizeof(uint2);
  const bool ok = L.D == 128 ? dispatch_kb<128>(L, grid, tab_bytes, st, k, v, slot_mapping, rows, pages)
                             : dispatch_kb<64>(L, grid, tab_bytes, st, k, v, slot_mapping, rows, pages);
  if (!ok) return (int)hipErrorInvalidValue;  // bit widths are validated by the API layer
  if (L.qjl) {
    const int rpw = kWG / (L.D / 8);
    const int64_t need = (rows + rpw - 1) / rpw;
    const dim3 qgrid((unsigned)(need < 65536 ? need : 65536));  // the kernel strides past the grid
    if (L.D == 128)
      hipLaunchKernelGGL(tq_qjl_kernel<128>, qgrid, dim3(kWG), 0, st, L, 1.0 / __builtin_sqrt(128.0),
                         (const uint16_t*)k, slot_mapping, rows, (uint8_t*)pages);
    else
      hipLaunchKernelGGL(tq_qjl_kernel<64>, qgrid, dim3(kWG), 0, st, L, 0.125,
                         (const uint16_t*)k, slot_mapping, rows, (uint8_t*)pages);
  }
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
