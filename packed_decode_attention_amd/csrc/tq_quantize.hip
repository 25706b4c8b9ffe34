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

#include "tq_device.h"

namespace {
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

// One region (K or V, BITS-bit codes) of the wave's 16 rows: norm, rotation, decisions, packing,
// store.  TABLE: decisions by the bucket table (resolution 2^sh), else by binary search.
// NC: norm-correction format (the stored norm is n / ||c[idx]||; s_c holds the centroids).
// MEAN: mean-removal format (the centred row is rotated; the mean is stored after the norm).
template <int D, int BITS, bool TABLE, bool NC, bool MEAN>
__device__ __forceinline__ void quantize_region(const uint4 (&x)[D / 32], const uint4 (&A)[D / 32][2],
                                                float zero, int g, int code_bytes,
                                                const float* s_t, const uint2* tab, int sh,
                                                const float* s_c, float rsqrt_d,
                                                uint8_t* __restrict__ dst) {
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
  // g < NB then holds the whole 4 BITS-byte run g (its pieces from lanes 0..3 in order) and stores
  // it in one or two instructions; then the norm.  Every lane stores (rows with no slot write to
  // the discard buffer), so a region issues a fixed number of stores.
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
  if (NB == 4 || g < NB) {
    uint8_t* run = dst + 4 * BITS * g;
    if constexpr (BITS == 8) {
      uint4* o = reinterpret_cast<uint4*>(run);
      o[0] = make_uint4(lo[0], hi[0], lo[1], hi[1]);
      o[1] = make_uint4(lo[2], hi[2], lo[3], hi[3]);
    } else if constexpr (BITS == 4) {
      *reinterpret_cast<uint4*>(run) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    } else if constexpr (BITS == 3) {  // four 24-bit pieces: 12 bytes
      *reinterpret_cast<uint3*>(run) = make_uint3(lo[0] | (lo[1] << 24), (lo[1] >> 8) | (lo[2] << 16),
                                                  (lo[2] >> 16) | (lo[3] << 8));
    } else {  // four 16-bit pieces: 8 bytes
      *reinterpret_cast<uint2*>(run) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
    }
  }
  if (g == 0) {
    if constexpr (MEAN)
      *reinterpret_cast<uint2*>(dst + code_bytes) = make_uint2(__float_as_uint(n_store), __float_as_uint(mu));
    else
      *reinterpret_cast<float*>(dst + code_bytes) = n_store;
  }
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
  // A operands: lane (row m = lane % 16, k = 8 (lane / 16) + j) of tile t holds
  // H_32[r][k] * s_{32 b + k} as fp16 +-1, r = 8 (m / 4) + 4 t + m % 4.  The sign of H_32[r][8 g + j]
  // is parity(r & 8 g) (one bit per lane) xor parity((r & 7) & j) (bit j of the 8-point Walsh row
  // r & 7, a byte of a 64-bit constant), and the sign flips of s are bits 8 g .. 8 g + 7 of the
  // block's sign word.
  constexpr uint64_t kWalsh8 = 0x963C5AF066CCAA00ull;  // byte x: bit j = parity(x & j)
  const uint32_t hpar = (__builtin_popcount((c >> 2) & g) & 1) ? 0xffu : 0u;
  uint4 A[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t x = ((uint32_t)(kWalsh8 >> (8 * (4 * t + (c & 3)))) & 0xffu) ^ hpar ^
                         ((L.signs.w[b] >> (8 * g)) & 0xffu);
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)  // fp16 +-1 pair: sign bits 2 q and 2 q + 1 of x
        w[q] = 0x3C003C00u | ((x << (15 - 2 * q)) & 0x8000u) | ((x << (30 - 2 * q)) & 0x80000000u);
      A[b][t] = make_uint4(w[0], w[1], w[2], w[3]);
      // computed here, while the codebook loads are in flight, not sunk past the table build
      asm volatile("" : "+v"(A[b][t].x), "+v"(A[b][t].y), "+v"(A[b][t].z), "+v"(A[b][t].w));
    }
  }
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
    int sh = gap > 0.0f ? -ilogbf(gap) : kQNoTable;  // bucket width 2^-sh <= gap
    if (sh < 0) sh = 0;
    if (gap <= 0.0f || 2 * (1 << min(sh, 20)) + 2 > qtab_entries(tid == 0 ? KB : VB)) sh = kQNoTable;
    s_sh[tid] = sh;
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

      quantize_region<D, KB, kTable, NC, MEAN>(xk, A, zero, g, L.kcode_bytes, s_t[0], tabk, shk,
                                               s_c[0], rsqrt_d, dst);
      quantize_region<D, VB, kTable, NC, MEAN>(xv, A, zero, g, L.vcode_bytes, s_t[1], tabv, shv,
                                               s_c[1], rsqrt_d, dst + L.kreg);
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
