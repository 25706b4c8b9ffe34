// Device helpers shared by the gfx950 kernels (tq_quantize.hip, tq_decode.hip).
//
// Lane layout used throughout: a (token, kv head) row of D coordinates is owned by a "row group"
// of consecutive lanes; lane j of a group of P lanes holds C = D/P consecutive coordinates
// C*j .. C*j + C - 1.  The Walsh-Hadamard transform of a row is then log2(C) in-register
// butterfly stages (coordinate bits below log2 C) followed by log2(P) cross-lane stages, and the
// packed codes of lane j are the C*bits/8 bytes starting at byte (C*bits/8)*j of the region.
#ifndef TQ_DEVICE_H_
#define TQ_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tqd {

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


// ---------------------------------------------------------------------------------------------
// Cross-lane data movement with DPP (no LDS traffic).  All patterns stay inside 8-lane groups.
// ---------------------------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppQuadRev = 0x1B;       // quad_perm [3,2,1,0]
constexpr int kDppHalfRowMirror = 0x141;  // lane i <- lane 7-i within each 8-lane half row
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within each 16-lane row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppRowRor8 = 0x128;        // lane i <- lane (i + 8) mod 16 within each 16-lane row

// x of lane (i XOR M) within each 16-lane row, M = 1, 2, 4 or 8, by one or two DPP moves.
template <int M>
__device__ __forceinline__ float dpp_xor(float x) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "DPP xor partner");
  if constexpr (M == 1) return dpp<kDppQuadXor1>(x);
  if constexpr (M == 2) return dpp<kDppQuadXor2>(x);
  if constexpr (M == 4) return dpp<kDppQuadRev>(dpp<kDppHalfRowMirror>(x));  // 7-i, then quad reversal
  return dpp<kDppRowRor8>(x);
}

// Walsh-Hadamard transform (Sylvester order) of a row of 8*P floats held by P <= 16 lanes of one
// DPP row, 8 per lane (lane j holds elements 8j .. 8j+7): in-lane butterflies, then DPP partners.
template <int P>
__device__ __forceinline__ void wht_row8_dpp(float (&x)[8], int j) {
#pragma unroll
  for (int hb = 1; hb < 8; hb <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!(e & hb)) {
        const float a = x[e], b = x[e | hb];
        x[e] = a + b;
        x[e | hb] = a - b;
      }
    }
  }
  auto level = [&](auto partner, int m) {
    const float sgn = (j & m) ? -1.0f : 1.0f;  // lower lane: x + p, upper lane: p - x
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(x[e], sgn, partner(x[e]));
  };
  if constexpr (P >= 2) level([](float v) { return dpp_xor<1>(v); }, 1);
  if constexpr (P >= 4) level([](float v) { return dpp_xor<2>(v); }, 2);
  if constexpr (P >= 8) level([](float v) { return dpp_xor<4>(v); }, 4);
  if constexpr (P >= 16) level([](float v) { return dpp_xor<8>(v); }, 8);
}

// Sum over aligned groups of P lanes (P = 1, 2, 4, 8, 16), result in every lane of the group.
template <int P>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (P >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (P >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (P >= 8) x += dpp<kDppHalfRowMirror>(x);
  if constexpr (P >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

// Walsh-Hadamard transform (Sylvester order) of a row held by P lanes x C values, lane j holding
// coordinates C*j .. C*j + C - 1.
template <int C, int P, typename T>
__device__ __forceinline__ void wht_row(T (&x)[C], int j) {
#pragma unroll
  for (int hb = 1; hb < C; hb <<= 1) {
#pragma unroll
    for (int e = 0; e < C; ++e) {
      if (!(e & hb)) {
        const T a = x[e], b = x[e | hb];
        x[e] = a + b;
        x[e | hb] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < P; m <<= 1) {
    const bool upper = (j & m) != 0;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      const T p = __shfl_xor(x[e], m, P);
      x[e] = upper ? p - x[e] : x[e] + p;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Packed codes of one lane: NB = C*bits/8 bytes at byte NB*j of a 4-byte aligned region, returned
// LSB-first in NW = ceil(NB/4) dwords.  Unaligned starts (bits 2 and 3) read the two dwords that
// cover them; the second one is at most the region's norm, so reads stay inside the slot.
// ---------------------------------------------------------------------------------------------
template <int NB>
struct LaneCodes {
  static constexpr int NW = (NB + 3) / 4;
  uint32_t w[NW];
};

template <int NB>
__device__ __forceinline__ LaneCodes<NB> load_lane_codes(const uint8_t* region, int j) {
  LaneCodes<NB> r;
  if constexpr (NB % 4 == 0) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(region + NB * j);
    if constexpr (NB == 4) {
      r.w[0] = p[0];
    } else if constexpr (NB == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      r.w[0] = v.x;
      r.w[1] = v.y;
    } else {
      static_assert(NB == 16, "unsupported lane code width");
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      r.w[0] = v.x;
      r.w[1] = v.y;
      r.w[2] = v.z;
      r.w[3] = v.w;
    }
  } else {
    static_assert(NB == 2 || NB == 3 || NB == 6, "unsupported lane code width");
    const int off = NB * j;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(region + (off & ~3));
    const uint32_t sh = (off & 3) * 8;
    const uint32_t u0 = p[0];
    const uint32_t u1 = (NB == 2) ? 0u : p[1];
    r.w[0] = __builtin_amdgcn_alignbit(u1, u0, sh);
    if constexpr (NB == 6) r.w[1] = u1 >> sh;
  }
  return r;
}

// ---------------------------------------------------------------------------------------------
// Centroid lookup tables in LDS, built from the fp32 codebook: one lookup per byte of codes
// (2-bit: 4 codes/byte -> float4, 4-bit: 2 codes -> float2, 8-bit: 1 code -> float), or per
// 6-bit pair of 3-bit codes (float2).
// ---------------------------------------------------------------------------------------------
template <int BITS>
struct Lut {
  static constexpr int kFloats = BITS == 2 ? 1024 : BITS == 3 ? 128 : BITS == 4 ? 512 : 256;
};

template <int BITS>
__device__ __forceinline__ void build_lut(float* t, const float* __restrict__ c, int tid, int nthreads) {
  for (int i = tid; i < Lut<BITS>::kFloats; i += nthreads) {
    float v;
    if constexpr (BITS == 2) v = c[((i >> 2) >> (2 * (i & 3))) & 3];
    else if constexpr (BITS == 3) v = c[((i >> 1) >> (3 * (i & 1))) & 7];
    else if constexpr (BITS == 4) v = c[((i >> 1) >> (4 * (i & 1))) & 15];
    else v = c[i];
    t[i] = v;
  }
}

// The C centroid values of one lane's codes.
template <int BITS, int C>
__device__ __forceinline__ void lookup_codes(const LaneCodes<C * BITS / 8>& code, const float* t,
                                             float (&out)[C]) {
  if constexpr (BITS == 3) {
    uint64_t u = code.w[0];
    if constexpr (C > 8) u |= (uint64_t)code.w[1] << 32;
#pragma unroll
    for (int g = 0; g < C / 2; ++g) {
      const uint32_t six = (uint32_t)(u >> (6 * g)) & 63u;
      const float2 v = reinterpret_cast<const float2*>(t)[six];
      out[2 * g] = v.x;
      out[2 * g + 1] = v.y;
    }
  } else {
    constexpr int PER = 8 / BITS;  // codes per byte
#pragma unroll
    for (int b = 0; b < C / PER; ++b) {
      const uint32_t byte = (code.w[b >> 2] >> (8 * (b & 3))) & 0xffu;
      if constexpr (BITS == 2) {
        const float4 v = reinterpret_cast<const float4*>(t)[byte];
        out[4 * b] = v.x;
        out[4 * b + 1] = v.y;
        out[4 * b + 2] = v.z;
        out[4 * b + 3] = v.w;
      } else if constexpr (BITS == 4) {
        const float2 v = reinterpret_cast<const float2*>(t)[byte];
        out[2 * b] = v.x;
        out[2 * b + 1] = v.y;
      } else {
        out[b] = t[byte];
      }
    }
  }
}

}  // namespace tqd

#endif  // TQ_DEVICE_H_
