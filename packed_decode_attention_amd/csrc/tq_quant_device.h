// Device code of the quantizer shared by the quantize-append kernel (tq_quantize.hip) and the
// fused append in the block decode kernel (tq_decode_block.hip): the rotation on the matrix cores,
// the norm tree, the bucket-table decisions and the packing of one region of 16 rows.
#ifndef TQ_QUANT_DEVICE_H_
#define TQ_QUANT_DEVICE_H_

#include "tq_device.h"

namespace tqq {
using namespace tqd;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// =============================================================================================
// Quantize-on-append
//
// A wave quantizes 16 rows (token, kv head) at a time, K then V.  Lane (g, c), g = lane / 16,
// c = lane % 16, loads coordinates 32 b + 8 g .. 32 b + 8 g + 7 of row c for every 32-coordinate
// block b (NB = D / 32 blocks, 16 bytes each): for each block this is the B operand of
// v_mfma_f32_16x16x32_f16, contraction index k = 8 g + j over the block's coordinates, one row
// per column.
//
// Rotation.  With i = 32 b + r the Sylvester Hadamard matrix factors as H_D = H_NB (x) H_32.  The
// matrix cores apply diag(s) followed by H_32 inside each block: the A operand holds the +-1
// entries of H_32 with the block's signs folded in, exact in fp16 like the fp16 inputs, so every
// product is exact and only the fp32 sums round.  A's rows are ordered so that result lane (g, c)
// receives rotated coordinates 8 g .. 8 g + 7 of each block of row c (rows 4 g .. 4 g + 3 of the
// result tile t hold 8 g + 4 t .. 8 g + 4 t + 3); H_NB across the blocks is then one or two
// butterfly levels inside the lane, and the lane's codes are NB runs of 8 consecutive coordinates.
//
// Norm.  Squares of fp16 values are exact in fp32 and the stride-halving tree (pairs i, i + D/2
// first, then D/4, ...) fixes every rounding.  The block index holds the top bits of i and sits
// inside the lane, so the first levels are in-lane (the first one fused with a square: one
// v_fma_mix each); bits 4 and 3 of i are bits 5 and 4 of the lane id and are reduced with
// permlane32 / permlane16 swaps, which exchange and transpose at once (each halves the values per
// lane); bits 2, 1, 0 follow in that order, spread over the lanes after the transposes.
//
// Decisions: idx = #{j : t_j <= u}.  With S a power of two no smaller than 1 / (smallest gap between
// boundaries), the bucket floor(u S) holds at most one boundary; a table gives per bucket the
// number of boundaries below it and the next boundary times S, so idx = base + (u S >= S t).  u S
// scales u exactly, so the decision is the comparison of u with the fp32 boundaries.  A codebook
// whose boundaries are closer than the table allows falls back to a binary search.
//
// Norm correction (tq-kv "How It Works": the quantiser's norm-correction stage and the corrected
// norm of its output record), a format flag: the stored norm is n / ||c[idx]|| so the dequantized
// row keeps norm n.  ||c[idx]||^2 follows the same tree over the rotated coordinates, on the fp32
// squares of the chosen centroids: the lane holds one code per block for the same low bits, so the
// block levels are in-lane again and the rest reuses the norm's swap network.
// =============================================================================================
constexpr int kQTabSmall = 130;   // bucket-table entries for codes of up to 4 bits (S <= 64)
constexpr int kQTabLarge = 2050;  // for 8-bit codes (S <= 1024)
constexpr int kQNoTable = -100;   // log2 S marker: binary search

__host__ __device__ constexpr int qtab_entries(int bits) { return bits <= 4 ? kQTabSmall : kQTabLarge; }

__device__ __forceinline__ float4_t mfma_f16_acc(const uint4& a, const uint4& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma_f16(const uint4& a, const uint4& b) {
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), zero, 0, 0, 0);
}

// fp16 number j (0..7) of an operand register quadruple, as fp32.
__device__ __forceinline__ float half_of(const uint4& v, int j) {
  const uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
  return half_bits_to_float((j & 1) ? (w >> 16) : (w & 0xffffu));
}

// Transpose-reduce across lanes l and l ^ 32 (M = 32) or l ^ 16 (M = 16): returns, in the lower
// lane of each pair, a(l) + a(partner), and in the upper lane b(partner) + b(l).
template <int M>
__device__ __forceinline__ float swap_add(float a, float b) {
  const auto r = M == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                         : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 4 x 4 transpose across the lane groups g = lane / 16: on return, lane group g holds in w[j]
// what lane group j held in w[g] (same lane within the group).  Exchanges across lane bit 5, then
// bit 4.
__device__ __forceinline__ void transpose_groups(uint32_t (&w)[4]) {
  auto swap32 = [](uint32_t& x, uint32_t& y) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    x = r[0];
    y = r[1];
  };
  auto swap16 = [](uint32_t& x, uint32_t& y) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    x = r[0];
    y = r[1];
  };
  swap32(w[0], w[2]);
  swap32(w[1], w[3]);
  swap16(w[0], w[1]);
  swap16(w[2], w[3]);
}

// The tree levels of coordinate bits 4 .. 0, given per lane the partial sums p[j] of coordinates
// with bits 0..2 = j and bits 3, 4 = this lane's g (bits 5, 6 already summed in-lane); the total
// ends up in every lane of the row.
__device__ __forceinline__ float tree_lanes(const float (&p)[8]) {
#pragma clang fp contract(off)
  // bit 4 (lane bit 5): q[j] = class (g & 1, j + 4 (g >> 1)) summed over bit 4
  float q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = swap_add<32>(p[j], p[j + 4]);
  // bit 3 (lane bit 4): t[j] = class j + 2 g (bits 0..2) summed over bits 3 and 4
  const float t0 = swap_add<16>(q[0], q[2]);
  const float t1 = swap_add<16>(q[1], q[3]);
  // bit 2: lanes g = 0, 1, 2, 3 hold classes 0, 2, 1, 3 of bits 0..1
  const float w = swap_add<32>(t0, t1);
  // bit 1: lanes g < 2 hold class 0 of bit 0, lanes g >= 2 class 1
  const float y = swap_add<16>(w, w);
  // bit 0
  return swap_add<32>(y, y);
}

// Sum of squares of a row by the stride-halving tree, in every lane of the row (see above).
template <int NB>
__device__ __forceinline__ float row_sum_squares(const uint4 (&x)[NB], float zero) {
#pragma clang fp contract(off)
  float p[8];  // partial sums of coordinates with bits 0..2 = j and bits 3, 4 = this lane's g
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (NB == 4) {  // pairs (b, b + 2), then (0, 1): bits 6 and 5 of i
      const float s0 = __builtin_fmaf(half_of(x[0], j), half_of(x[0], j),
                                      __builtin_fmaf(half_of(x[2], j), half_of(x[2], j), zero));
      const float s1 = __builtin_fmaf(half_of(x[1], j), half_of(x[1], j),
                                      __builtin_fmaf(half_of(x[3], j), half_of(x[3], j), zero));
      p[j] = s0 + s1;
    } else {  // pair (0, 1): bit 5 of i
      p[j] = __builtin_fmaf(half_of(x[0], j), half_of(x[0], j),
                            __builtin_fmaf(half_of(x[1], j), half_of(x[1], j), zero));
    }
  }
  return tree_lanes(p);
}

// The same tree over fp32 values v[b][j] at coordinates 32 b + 8 g + j: squares rounded to fp32.
template <int NB>
__device__ __forceinline__ float row_sum_squares_f32(const float (&v)[NB][8]) {
#pragma clang fp contract(off)
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (NB == 4) {
      const float s0 = v[0][j] * v[0][j] + v[2][j] * v[2][j];
      const float s1 = v[1][j] * v[1][j] + v[3][j] * v[3][j];
      p[j] = s0 + s1;
    } else {
      p[j] = v[0][j] * v[0][j] + v[1][j] * v[1][j];
    }
  }
  return tree_lanes(p);
}

// fp16 high and low parts of x: hi = fp16(x), lo = fp16(x - hi).
__device__ __forceinline__ void split_half(float x, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = (_Float16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)h));
}

// Mean-removal format: the row mean mu (the stride-halving fp32 tree of the values over D, an
// exact power-of-two scaling), the norm of the centred row d = fp32(x - mu) (squares rounded to
// fp32, the same tree) and d as fp16 high and low parts for the matrix cores: products with the
// +-1 operand stay exact and hi + lo carries d to about 22 bits, far inside the tie band.
template <int NB>
__device__ __forceinline__ void centre_row(const uint4 (&x)[NB], float& mu, float& n,
                                           uint4 (&xh)[NB], uint4 (&xl)[NB]) {
#pragma clang fp contract(off)
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (NB == 4) {
      p[j] = (half_of(x[0], j) + half_of(x[2], j)) + (half_of(x[1], j) + half_of(x[3], j));
    } else {
      p[j] = half_of(x[0], j) + half_of(x[1], j);
    }
  }
  mu = tree_lanes(p) * (1.0f / (32 * NB));
  float d[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 8; ++j) d[b][j] = half_of(x[b], j) - mu;
  n = sqrtf(row_sum_squares_f32<NB>(d));
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split_half(d[b][j], h[j], l[j]);
    xh[b] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    xl[b] = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
  }
}

// What one lane stores for one region of its row: the packed run it owns (4 BITS bytes: two
// 16-byte pieces at 8 bits, 16, 12 or 8 bytes below), the stored norm and, in the mean-removal
// format, the mean.
template <int BITS>
struct RegionBits {
  uint32_t w[BITS == 8 ? 8 : BITS == 4 ? 4 : BITS == 3 ? 3 : 2];
  float n_store, mu;
};

// Stores of one region: lane g < NB its run, lane 0 of the row the norm (and mean).  Every lane
// stores (rows with no slot write to the discard buffer), so a region issues a fixed number of
// stores: region_stores(BITS).
template <int D, int BITS, bool MEAN>
__device__ __forceinline__ void store_region(const RegionBits<BITS>& r, int g, int code_bytes,
                                             uint8_t* __restrict__ dst) {
  constexpr int NB = D / 32;
  if (NB == 4 || g < NB) {
    uint8_t* run = dst + 4 * BITS * g;
    if constexpr (BITS == 8) {
      uint4* o = reinterpret_cast<uint4*>(run);
      o[0] = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
      o[1] = make_uint4(r.w[4], r.w[5], r.w[6], r.w[7]);
    } else if constexpr (BITS == 4) {
      *reinterpret_cast<uint4*>(run) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    } else if constexpr (BITS == 3) {
      *reinterpret_cast<uint3*>(run) = make_uint3(r.w[0], r.w[1], r.w[2]);
    } else {
      *reinterpret_cast<uint2*>(run) = make_uint2(r.w[0], r.w[1]);
    }
  }
  if (g == 0) {
    if constexpr (MEAN)
      *reinterpret_cast<uint2*>(dst + code_bytes) = make_uint2(__float_as_uint(r.n_store), __float_as_uint(r.mu));
    else
      *reinterpret_cast<float*>(dst + code_bytes) = r.n_store;
  }
}

// One region (K or V, BITS-bit codes) of the wave's 16 rows: norm, rotation, decisions, packing;
// the lane's share of the stores is returned (store_region writes it).  TABLE: decisions by the
// bucket table (resolution 2^sh), else by binary search.
// NC: norm-correction format (the stored norm is n / ||c[idx]||; s_c holds the centroids).
// MEAN: mean-removal format (the centred row is rotated; the mean is stored after the norm).
template <int D, int BITS, bool TABLE, bool NC, bool MEAN>
__device__ __forceinline__ RegionBits<BITS> quantize_region_bits(const uint4 (&x)[D / 32],
                                                                 const uint4 (&A)[D / 32][2], float zero,
                                                                 const float* __restrict__ s_t,
                                                                 const uint2* __restrict__ tab, int sh,
                                                                 const float* __restrict__ s_c, float rsqrt_d) {
  constexpr int NB = D / 32;
  float n, mu = 0.0f;
  uint4 xh[NB], xl[NB];
  if constexpr (MEAN) centre_row<NB>(x, mu, n, xh, xl);
  else n = sqrtf(row_sum_squares<NB>(x, zero));  // correctly rounded

  // H_NB across blocks, scaled to u S = y S / (sqrt(D) n) (u = 0 for a zero row), and decisions.
  const float inv = n > 0.0f ? (TABLE ? ldexpf(rsqrt_d / n, sh) : rsqrt_d / n) : 0.0f;
  const uint2* tabp = tab + (TABLE ? (1 << sh) + 1 : 0);
  uint32_t code[NB][8];  // code[a][e]: rotated coordinate 32 a + 8 g + e
  float csq[8];          // NC: the in-lane tree levels (coordinate bits 6, 5) of fp32(c[code]^2)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float4_t z[NB];  // z[b][i]: H_32 diag(s) of block b at rotated coordinate 8 g + 4 t + i
#pragma unroll
    for (int b = 0; b < NB; ++b)
      z[b] = MEAN ? mfma_f16_acc(A[b][t], xl[b], mfma_f16(A[b][t], xh[b])) : mfma_f16(A[b][t], x[b]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) y[b] = z[b][i] * inv;
      if constexpr (NB == 4) {
        const float a0 = y[0] + y[1], a1 = y[0] - y[1], a2 = y[2] + y[3], a3 = y[2] - y[3];
        y[0] = a0 + a2;
        y[1] = a1 + a3;
        y[2] = a0 - a2;
        y[3] = a1 - a3;
      } else {
        const float a0 = y[0] + y[1], a1 = y[0] - y[1];
        y[0] = a0;
        y[1] = a1;
      }
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        const float us = y[a];
        if constexpr (TABLE) {
          const uint2 ent = tabp[(int)floorf(us)];
          code[a][4 * t + i] = ent.y + (us >= __uint_as_float(ent.x) ? 1u : 0u);
        } else {
          int id = 0;
#pragma unroll
          for (int st = (1 << BITS) >> 1; st >= 1; st >>= 1)
            if (s_t[id + st - 1] <= us) id += st;
          code[a][4 * t + i] = (uint32_t)id;
        }
      }
      if constexpr (NC) {
#pragma clang fp contract(off)
        float cv[NB];
#pragma unroll
        for (int a = 0; a < NB; ++a) cv[a] = s_c[code[a][4 * t + i]];
        if constexpr (NB == 4) {
          csq[4 * t + i] = (cv[0] * cv[0] + cv[2] * cv[2]) + (cv[1] * cv[1] + cv[3] * cv[3]);
        } else {
          csq[4 * t + i] = cv[0] * cv[0] + cv[1] * cv[1];
        }
      }
    }
  }
  // Stored norm: n, or with norm correction n / ||c[idx]|| (correctly rounded sqrt and division).
  float n_store = n;
  if constexpr (NC) {
    const float r = sqrtf(tree_lanes(csq));
    n_store = n > 0.0f ? n / r : 0.0f;
  }

  // Pack: run a (the lane's 8 codes at rotated coordinates 32 a + 8 g ..) is bytes BITS (4 a + g)
  // .. BITS (4 a + g + 1) - 1 of the region.  The four lanes of a row transpose their runs, so lane
  // g < NB then holds the whole 4 BITS-byte run g (its pieces from lanes 0..3 in order).
  uint32_t lo[4], hi[4];  // per run: the piece's bits (lo) and, for 8-bit codes, its upper dword
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    lo[a] = 0;
    hi[a] = 0;
    if (a < NB) {
      if constexpr (BITS == 8) {
        lo[a] = code[a][0] | (code[a][1] << 8) | (code[a][2] << 16) | (code[a][3] << 24);
        hi[a] = code[a][4] | (code[a][5] << 8) | (code[a][6] << 16) | (code[a][7] << 24);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[a] |= code[a][e] << (BITS * e);
      }
    }
  }
  transpose_groups(lo);
  if constexpr (BITS == 8) transpose_groups(hi);
  RegionBits<BITS> r;
  r.n_store = n_store;
  r.mu = mu;
  if constexpr (BITS == 8) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      r.w[2 * a] = lo[a];
      r.w[2 * a + 1] = hi[a];
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int a = 0; a < 4; ++a) r.w[a] = lo[a];
  } else if constexpr (BITS == 3) {  // four 24-bit pieces: 12 bytes
    r.w[0] = lo[0] | (lo[1] << 24);
    r.w[1] = (lo[1] >> 8) | (lo[2] << 16);
    r.w[2] = (lo[2] >> 16) | (lo[3] << 8);
  } else {  // four 16-bit pieces: 8 bytes
    r.w[0] = lo[0] | (lo[1] << 16);
    r.w[1] = lo[2] | (lo[3] << 16);
  }
  return r;
}

// One region quantized and stored at once.
template <int D, int BITS, bool TABLE, bool NC, bool MEAN>
__device__ __forceinline__ void quantize_region(const uint4 (&x)[D / 32], const uint4 (&A)[D / 32][2],
                                                float zero, int g, int code_bytes,
                                                const float* s_t, const uint2* tab, int sh,
                                                const float* s_c, float rsqrt_d,
                                                uint8_t* __restrict__ dst) {
  const RegionBits<BITS> r = quantize_region_bits<D, BITS, TABLE, NC, MEAN>(x, A, zero, s_t, tab, sh, s_c, rsqrt_d);
  store_region<D, BITS, MEAN>(r, g, code_bytes, dst);
}

// Bucket table of one codebook (see above), entries i0 .. i0 + kPer - 1 of this thread: entry
// {S t_base as bits, base} with base = #{t < k / S} for bucket k = i - (S + 1).  base0 is the
// entry i0's count.  Boundary base0 + m lies in bucket k0 + d_m (k0 = i0 - (S + 1), d_m >= m, the
// d_m distinct: one boundary per bucket at most), and it is below the edge of entry i0 + r exactly
// when d_m < r.  So with M the bit set of the d_m, entry i0 + r counts base0 + popcount(M below
// bit r).
template <int BITS, int kPer>
__device__ __forceinline__ void fill_qtab(const float* s_t, int sh, int i0, int base0, uint2* tab) {
  constexpr int nb = (1 << BITS) - 1;
  constexpr int kW = kPer > 1 ? kPer - 1 : 1;
  const bool valid = sh != kQNoTable;
  const int S = valid ? 1 << sh : 0;
  const int k0 = i0 - (S + 1);
  // (the empty asm statements keep each group of LDS reads unconditional and in flight together)
  float tb[kW];
#pragma unroll
  for (int m = 0; m + 1 < kPer; ++m) tb[m] = s_t[min(base0 + m, nb - 1)];
#pragma unroll
  for (int m = 0; m + 1 < kPer; ++m) asm volatile("" : "+v"(tb[m]));
  uint32_t M = 0;
#pragma unroll
  for (int m = 0; m + 1 < kPer; ++m) {
    const int d = base0 + m < nb ? min((int)floorf(ldexpf(tb[m], sh)) - k0, 31) : 31;
    M |= 1u << d;
  }
  int cnt[kPer];
  float nx[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    cnt[r] = base0 + __builtin_popcount(M & ((1u << r) - 1u));
    nx[r] = s_t[min(cnt[r], nb - 1)];
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) asm volatile("" : "+v"(nx[r]));
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    if (valid && i0 + r < 2 * S + 2) {
      const float next = cnt[r] < nb ? ldexpf(nx[r], sh) : 3.0e38f;
      tab[i0 + r] = make_uint2(__float_as_uint(next), (uint32_t)cnt[r]);
    }
  }
}

// Bucket tables of the K and V codebooks: each thread takes consecutive entries (up to nine per
// table), finds the count of its first entry by a branchless lower-bound search over the sorted
// boundaries (both tables' searches advance together), and derives the rest from the next few
// boundaries, so the build takes a few LDS round trips rather than one search per entry.
template <int KB, int VB>
__device__ __forceinline__ void build_qtabs(const float (*s_t)[256], int shk, int shv, uint2* tabk,
                                            uint2* tabv, int tid) {
  constexpr int kPK = (qtab_entries(KB) + kWG - 1) / kWG;  // entries per thread at most
  constexpr int kPV = (qtab_entries(VB) + kWG - 1) / kWG;
  constexpr int kStK = 1 << (KB - 1), kStV = 1 << (VB - 1);  // first step: nb = 2 st - 1
  constexpr int kSt0 = kStK > kStV ? kStK : kStV;
  const int i0k = tid * kPK, i0v = tid * kPV;
  auto edge0 = [](int i0, int sh) {
    return sh == kQNoTable ? 0.0f : ldexpf((float)(i0 - ((1 << sh) + 1)), -sh);
  };
  const float ek = edge0(i0k, shk), ev = edge0(i0v, shv);
  int bk = 0, bv = 0;
  // after the steps above st, a count is <= 2 st0 - 2 st, so count + st <= nb: every read is a
  // boundary
#pragma unroll
  for (int st = kSt0; st >= 1; st >>= 1) {
    if (st <= kStK) {
      const int j = bk + st;
      bk = s_t[0][j - 1] < ek ? j : bk;
    }
    if (st <= kStV) {
      const int j = bv + st;
      bv = s_t[1][j - 1] < ev ? j : bv;
    }
  }
  asm volatile("" : "+v"(bk), "+v"(bv));  // both searches above, interleaved
  fill_qtab<KB, kPK>(s_t[0], shk, i0k, bk, tabk);
  fill_qtab<VB, kPV>(s_t[1], shv, i0v, bv, tabv);
}

// Hadamard A operands: lane (row m = lane % 16, k = 8 (lane / 16) + j) of tile t holds
// H_32[r][k] * s_{32 b + k} as fp16 +-1, r = 8 (m / 4) + 4 t + m % 4.  The sign of H_32[r][8 g + j]
// is parity(r & 8 g) (one bit per lane) xor parity((r & 7) & j) (bit j of the 8-point Walsh row
// r & 7, a byte of a 64-bit constant), and the sign flips of s are bits 8 g .. 8 g + 7 of the
// block's sign word.
template <int NB>
__device__ __forceinline__ void hadamard_operands(const TqSigns& signs, int lane, uint4 (&A)[NB][2]) {
  const int c = lane & 15, g = lane >> 4;
  constexpr uint64_t kWalsh8 = 0x963C5AF066CCAA00ull;  // byte x: bit j = parity(x & j)
  const uint32_t hpar = (__builtin_popcount((c >> 2) & g) & 1) ? 0xffu : 0u;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t x = ((uint32_t)(kWalsh8 >> (8 * (4 * t + (c & 3)))) & 0xffu) ^ hpar ^
                         ((signs.w[b] >> (8 * g)) & 0xffu);
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)  // fp16 +-1 pair: sign bits 2 q and 2 q + 1 of x
        w[q] = 0x3C003C00u | ((x << (15 - 2 * q)) & 0x8000u) | ((x << (30 - 2 * q)) & 0x80000000u);
      A[b][t] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// log2 S of a codebook's bucket table (bucket width 2^-sh <= the smallest boundary gap), or
// kQNoTable when the gap is too fine for a table of its entries
__device__ __forceinline__ int qtab_shift(float gap, int bits) {
  int sh = gap > 0.0f ? -ilogbf(gap) : kQNoTable;
  if (sh < 0) sh = 0;
  if (gap <= 0.0f || 2 * (1 << min(sh, 20)) + 2 > qtab_entries(bits)) sh = kQNoTable;
  return sh;
}

}  // namespace tqq

#endif  // TQ_QUANT_DEVICE_H_
