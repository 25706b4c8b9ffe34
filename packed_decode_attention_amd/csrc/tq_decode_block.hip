// Fused paged decode attention over packed TQ pages, whole-block streaming kernel (gfx950), for
// the K4/V4 page format at D = 128 with eight kv heads of unpadded 136-byte slots, one codebook
// for keys and values, and up to four query heads per kv head (the Llama-3-8B-shaped workload).
//
// Method as in tq_decode.hip: scores on the codes with a rotated query, online softmax, values
// summed in the rotated frame, split-K partials merged by tq_decode_merge_kernel (tq-kv, "Custom
// CUDA Kernel Stack": split-KV flash decode on compressed KV; turboquant-pro 1.4.2, "Fused CUDA
// decode": split-K decode on the codes).  What differs is how page bytes reach the matrix cores:
//  * One persistent workgroup of 8 waves per compute unit takes (sequence, split) units in turn;
//    wave h computes kv head h.  The workgroup reads whole page runs (16 positions x 8 heads =
//    17 KB contiguous): each load instruction moves 1 KB of page bytes straight into LDS
//    (buffer_load ... lds), in a ring of five run buffers (four in flight while one is read).
//    Fetching one kv head's 136-byte rows instead (1088 bytes apart) streams about a quarter
//    slower on this chip.
//  * LDS reads are free of bank conflicts.  The loads place the 16-byte chunks of a run rotated
//    by (token / 4) within each aligned group of 16 chunks (the loads choose their source chunks,
//    the LDS side stays contiguous), so the 16 tokens of a run, 1088 bytes apart, no longer fall
//    on 4 banks.  The centroid operand table (one code byte -> fp16 high and low parts of its two
//    centroids, 8 bytes) is held in 32 interleaved copies, lane l reading copy l mod 32: the 32
//    lanes of each LDS pass read distinct bank pairs.  Its byte address (code << 8 | 8 copy) is
//    one v_perm of the code word.
//  * QK on v_mfma_f32_16x16x32_f16: rows are (query head, fp16 part of the query), columns the 16
//    tokens, K the coordinates with both fp16 parts of each centroid.  PV: rows are (query head,
//    fp16 part of the weight, nibble of the code byte), columns the code bytes of a dword (two
//    coordinates each), K the tokens with both centroid parts; every row is live, and the code
//    byte of one token indexes the table directly.
//  * Software pipeline: each step issues the next run's key lookups, then does the current run's
//    softmax and PV, then the next run's QK.  The running maxima are rescaled lazily (only when a
//    run's maximum exceeds the reference by more than one, in log2 units), which keeps the step
//    one basic block in the common case.

#include <climits>

#include "tq_device.h"

namespace {
using namespace tqd;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // one 8-byte LDS read

constexpr int kW = 8;                          // waves per workgroup: one per kv head
constexpr int kT = kW * 64;                    // threads per workgroup
constexpr int kH = 8;                          // kv heads
constexpr int kD = 128;
constexpr int kSB = 136;                       // slot bytes: K codes, K norm, V codes, V norm
constexpr int kVOff = 68;                      // V region offset in a slot
constexpr int kRowBytes = kH * kSB;            // one position, every kv head: 1088
constexpr int kRunBytes = 16 * kRowBytes;      // one run of 16 positions: 17408
constexpr int kWaveChunks = kRunBytes / 16 / kW;  // 16-byte chunks of a run each wave loads: 136
constexpr int kRing = 5;                       // run buffers
constexpr int kCP = 32;                        // table copies
constexpr int kLutShift = 8;                   // table entries hold c * 2^8
constexpr int kWShift = 13;                    // weights enter PV as w * 2^13 (below 2^15)
constexpr float kThr = 2.0f;                   // lazy rescale threshold, log2 units
constexpr float kSent = -1.0e30f;              // finite minus infinity of the running maxima
constexpr int kMaxRuns = 192;                  // runs per unit (three lanes' worth of run rows)
constexpr int kBuf0 = 256 * kCP * 8;           // first run buffer, after the 64 KB table
constexpr int kLdsBytes = kBuf0 + kRing * kRunBytes;

__device__ __forceinline__ float4_t mfma16(const uint4& a, const uint4& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                c, 0, 0, 0);
}

// fp16 high and low parts of x: hi = fp16(x), lo = fp16(x - hi).
__device__ __forceinline__ void split_half(float x, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = (_Float16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)h));
}

__device__ __forceinline__ float max16(float x) {  // maximum over a 16-lane row, in every lane
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppHalfRowMirror>(x));
  return fmaxf(x, dpp<kDppRowMirror>(x));
}

__device__ __forceinline__ float lane_value(float x, int l) {  // x of lane l, wave-uniform
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Workgroup barrier that completes this wave's LDS operations only: run loads in flight stay in
// flight (a release fence would also drain them, as they write LDS).  The memory clobber keeps the
// compiler from moving any memory access across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier that leaves this wave's LDS reads in flight (table lookups that read no run
// buffer).  Used where every read of the run buffer released by the barrier has already been
// consumed, so its data is in registers.
__device__ __forceinline__ void step_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate leaving n vector memory operations outstanding (gfx9 encoding).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xf00; }

// A wave-uniform read of memory the kernel never writes, as a scalar load.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(reinterpret_cast<uintptr_t>(p));
}

// Raw buffer resource over n bytes from p (out-of-range reads return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// 16 bytes per lane from byte off of a buffer straight into LDS: lane l writes dst + 16 l (dst
// wave-uniform).  The buffer form of the LDS load keeps the compiler's LDS waits counted (it
// forces every LDS wait to zero while a global-address LDS load is in flight).
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, lds_u8* dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ lds_u8* lds_ptr(uint8_t* p) { return (lds_u8*)p; }

// LDS placement of a run: byte g of the run (position g / 1088, slot byte g mod 1088) sits in
// chunk slot ((g / 16 + q) mod 16) of its aligned group of 16 chunks, q = g / 4352 (the token's
// index divided by four).  A group never straddles two values of q (4352 bytes = 17 groups).
__device__ __forceinline__ int run_lds_offset(int g) {
  const int c = g >> 4, q = c / 272;
  return (((c & ~15) | ((c + q) & 15)) << 4) | (g & 15);
}
// The run chunk that LDS chunk p holds (the inverse of the placement above).
__device__ __forceinline__ int run_chunk_at(int p) {
  const int q = p / 272;
  return (p & ~15) | ((p - q) & 15);
}

}  // namespace

struct TqBlockArgs {
  const uint16_t* q;
  const uint8_t* pages;
  const int32_t* bt;
  const int32_t* seq_lens;
  const int32_t* win_lens;  // NULL: no hot window
  float* partials;          // [B][8][part_stride][G][D + 2]
  const float* c;           // the codebook of keys and values (16 centroids)
  TqSigns signs;
  float qscale;             // scale * log2(e) / sqrt(D)
  int max_blocks, bs, bs_shift, G, Hq, n_sink, win_cap;
  int chunk, max_split, part_stride, n_units;
  int nq, q0, g_real;       // several queries per sequence (one: 1, 0, G)
};

namespace {

__device__ __forceinline__ int64_t q_row(const TqBlockArgs& a, int b, int h, int v) {
  const int jq = v / a.g_real;
  return ((int64_t)b * a.nq + a.q0 + jq) * a.Hq + (int64_t)h * a.g_real + (v - jq * a.g_real);
}

// Page row (block id * bs + offset in the block) of the first position of run r of sequence b.
__device__ __forceinline__ int run_row(const TqBlockArgs& a, int b, int r) {
  const int pos = 16 * r;
  const int blk = a.bs_shift >= 0 ? (pos >> a.bs_shift) : (pos / a.bs);
  return a.bt[(int64_t)b * a.max_blocks + blk] * a.bs + (pos - blk * a.bs);
}

// Unit bookkeeping shared by the producer and the compute waves (every wave takes the same
// branches, so the workgroup barriers match).
struct TqUnit {
  int b, split, seq_len, ns, end, run0, n_run;
  bool live;  // false: no partial is read for this split
};

__device__ __forceinline__ TqUnit unit_of(const TqBlockArgs& a, int unit) {
  TqUnit u;
  u.b = unit / a.max_split;
  u.split = unit - u.b * a.max_split;
  u.seq_len = load_uniform(a.seq_lens + u.b);
  u.ns = min(a.n_sink, u.seq_len);
  int win = 0;
  if (a.win_lens != nullptr) win = max(0, min(load_uniform(a.win_lens + u.b), min(a.win_cap, u.seq_len - u.ns)));
  const int packed_end = u.seq_len - win;
  const int nsplit = packed_end > 0 ? (packed_end + a.chunk - 1) / a.chunk : 1;
  u.live = u.split < nsplit;  // the merge reads the partials of splits below nsplit only
  const int start = u.split * a.chunk;
  u.end = min(start + a.chunk, packed_end);
  // Positions from the run holding the first non-sink position; rows below ns are masked, runs of
  // sinks only are never read.
  const int p0 = max(start, u.ns & ~15);
  const bool any = u.end > max(p0, u.ns);
  u.run0 = p0 >> 4;
  u.n_run = any ? ((u.end - 1) >> 4) - u.run0 + 1 : 0;
  return u;
}

__global__ __launch_bounds__(kT + 256) void tq_decode_block_kernel(TqBlockArgs a) {
  // One LDS array placed by hand: the table at byte 0, run buffer k at kBuf0 + 17408 k.  Only the
  // producer wave has loads in flight, and it reads no LDS, so the compute waves' reads need no
  // alias information to stay clear of pending loads.
  __shared__ __align__(16) uint8_t s_lds[kLdsBytes];
  uint2* const s_tab = reinterpret_cast<uint2*>(s_lds);
  uint8_t* const s_r0 = s_lds + kBuf0;
  uint8_t* const s_r1 = s_r0 + kRunBytes;
  uint8_t* const s_r2 = s_r1 + kRunBytes;
  uint8_t* const s_r3 = s_r2 + kRunBytes;
  uint8_t* const s_r4 = s_r3 + kRunBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7: kv head; 8..11: run loads
  const int t16 = lane & 15, q4 = lane >> 4;
  const int G = a.G;

  // Centroid operand table: entry e (a code byte: coordinates 2j, 2j + 1 in its low and high
  // nibble) holds the fp16 high parts of c[e & 15], c[e >> 4], then their low parts, scaled by
  // 2^8; copy k of entry e at byte 256 e + 8 k.
  for (int i = tid; i < 256 * kCP; i += kT + 256) {
    const int e = i / kCP;
    uint32_t h0, l0, h1, l1;
    split_half(ldexpf(a.c[e & 15], kLutShift), h0, l0);
    split_half(ldexpf(a.c[e >> 4], kLutShift), h1, l1);
    s_tab[i] = make_uint2(h0 | (h1 << 16), l0 | (l1 << 16));
  }
  // The run buffers are written by the loads (which the compiler does not see as stores): one
  // ordinary store keeps it from treating the array as never written there.
  if (tid == 0) s_r0[0] = 0;

  if (wave >= kW) {
    // ======== producer waves: every page load of the workgroup ========
    // Run r goes to buffer r mod 5 in 17 loads of 1 KB (LDS chunks 64 k + lane); producer p issues
    // loads k = p, p + 4, ... of every run.  One wave issues such loads at about a fifth of the
    // rate the memory system serves a compute unit, so a run's loads are spread over four waves.
    // While the compute waves read run s + 1, runs s + 2 .. s + 5 are in flight.  The compute
    // waves never issue a vector memory instruction in the loop, so a busy load path stalls these
    // waves only.
    const int pw = wave - kW;           // producer 0..3
    const int nk = pw == 0 ? 5 : 4;     // loads per run of this producer
    int src_off[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) src_off[i] = 16 * run_chunk_at(64 * min(pw + 4 * i, 16) + lane);
    for (int unit = blockIdx.x; unit < a.n_units; unit += gridDim.x) {
      const TqUnit u = unit_of(a, unit);
      if (!u.live) continue;
      const int n_run = u.n_run;
      lds_barrier();  // every wave is done with the previous unit's buffers
      // page rows of runs run0 + lane, + 64, + 128 (clamped to the last run)
      int rows0 = 0, rows1 = 0, rows2 = 0;
      if (n_run > 0) {
        rows0 = run_row(a, u.b, u.run0 + min(lane, n_run - 1));
        rows1 = run_row(a, u.b, u.run0 + min(lane + 64, n_run - 1));
        rows2 = run_row(a, u.b, u.run0 + min(lane + 128, n_run - 1));
      }
      auto issue = [&](int r, lds_u8* buf) {
        const int row = r < 64 ? __builtin_amdgcn_readlane(rows0, r)
                               : r < 128 ? __builtin_amdgcn_readlane(rows1, r - 64)
                                         : __builtin_amdgcn_readlane(rows2, r - 128);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.pages + (int64_t)row * kRowBytes, kRunBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16(rs, buf + 1024 * (pw + 4 * i), src_off[i]);
        if (pw == 0) lds_dma16(rs, buf + 1024 * 16, src_off[4]);
      };
      // wait for this wave's loads of run r, with those of the later runs (up to three) in flight
      auto wait_run = [&](int r) {
        const int later = min(n_run - 1, r + 3) - r;
        if (later >= 3) {
          if (pw == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(15));
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
        } else if (later == 2) {
          if (pw == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(10));
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
        } else if (later == 1) {
          if (pw == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(5));
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
      };
      (void)nk;
      // runs 0..3 (buffer 4 holds the compute waves' queries until the first barrier)
      if (n_run > 0) issue(0, lds_ptr(s_r0));
      if (n_run > 1) issue(1, lds_ptr(s_r1));
      if (n_run > 2) issue(2, lds_ptr(s_r2));
      if (n_run > 3) issue(3, lds_ptr(s_r3));
      if (n_run <= 0) continue;
      // run 0 is in (runs 1..3 may be in flight; run 4 is not issued yet)
      {
        const int later = min(n_run - 1, 3);
        if (later >= 3) {
          if (pw == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(15));
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
        } else if (later == 2) {
          if (pw == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(10));
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
        } else if (later == 1) {
          if (pw == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(5));
          else __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
      }
      lds_barrier();
      if (n_run > 4) issue(4, lds_ptr(s_r4));
      // step s: every producer waits for its loads of run s + 1, barrier (every wave is done with
      // run s), then they fetch run s + 5 into run s's buffer
      auto step = [&](int s, lds_u8* fill) {
        if (s + 1 < n_run) wait_run(s + 1);
        lds_barrier();
        if (s + 5 < n_run) issue(s + 5, fill);
      };
      for (int s = 0; s < n_run; s += kRing) {
        step(s, lds_ptr(s_r0));
        if (s + 1 < n_run) step(s + 1, lds_ptr(s_r1));
        if (s + 2 < n_run) step(s + 2, lds_ptr(s_r2));
        if (s + 3 < n_run) step(s + 3, lds_ptr(s_r3));
        if (s + 4 < n_run) step(s + 4, lds_ptr(s_r4));
      }
    }
    return;
  }

  // ======== compute waves: wave h computes kv head h ========
  const int h = wave;
  const uint8_t* const tab = reinterpret_cast<const uint8_t*>(s_tab);
  const uint32_t kcopy = 8u * (uint32_t)(lane & 31);

  // ---- per-lane LDS offsets within a run buffer (the same for every run) ----
  // K codes of token t16, bytes 16 q4 .. 16 q4 + 15 of the K region, as two 8-byte reads; lanes
  // with odd q4 read the upper half first (the two halves of a 32-lane pass then use distinct
  // banks).  Word order: w[0..1] = first read, w[2..3] = second.
  // Each offset is held as an LDS address less 64 KB (opaque to the compiler), so a read adds the
  // buffer's base minus 64 KB as the DS instruction's immediate offset: no address arithmetic
  // per read for the four buffers whose base is below 128 KB.
  auto lane_addr = [](int off) {
    int x = off + kBuf0;
    asm volatile("" : "+v"(x));
    return x;
  };
  const int sw = q4 & 1;
  const int kbase = kRowBytes * t16 + kSB * h + 16 * q4;
  const int off_k0 = lane_addr(run_lds_offset(kbase + 8 * sw));
  const int off_k1 = lane_addr(run_lds_offset(kbase + 8 * (1 - sw)));
  const int off_kn = lane_addr(run_lds_offset(kRowBytes * t16 + kSB * h + 64));
  const int off_vn = lane_addr(run_lds_offset(kRowBytes * t16 + kSB * h + kVOff + 64));
  // V codes: dword t16 (coordinates 8 t16 .. 8 t16 + 7) of tokens q4 + 4 m, m = 0..3
  int off_v[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    off_v[m] = lane_addr(run_lds_offset(kRowBytes * (q4 + 4 * m) + kSB * h + kVOff + 4 * t16));
  // read of buffer `buf` at lane address x
  auto at = [&](const uint8_t* buf, int x) { return buf - kBuf0 + x; };
  // PV weight gather: row t16 of the A operand is (head t16 >> 2, nibble (t16 >> 1) & 1, weight
  // part t16 & 1); it takes the weights of tokens q4 + 4 m from softmax lane 16 (t16 >> 2) + token.
  const int bp_base = 4 * (16 * (t16 >> 2) + q4);
  const uint32_t bp_sel = ((t16 >> 1) & 1) ? ((t16 & 1) ? 0x03020c0cu : 0x01000c0cu)
                                           : ((t16 & 1) ? 0x0c0c0302u : 0x0c0c0100u);

  for (int unit = blockIdx.x; unit < a.n_units; unit += gridDim.x) {
    const TqUnit u = unit_of(a, unit);
    if (!u.live) continue;
    const int b = u.b, n_run = u.n_run, run0 = u.run0;

    lds_barrier();  // every wave is done with the previous unit's buffers

    // This wave's fp16 queries (4 rows of 256 bytes) into its 2176-byte region of buffer 4, which
    // takes a run only after the first step's barrier.
    uint8_t* const qreg = s_r4 + h * (kWaveChunks * 16);
    {
      const int g = q4 < G ? q4 : 0;  // query heads past G read a live row, unused
      const int64_t r0q = q_row(a, b, h, 0);
      const int dq = (int)(q_row(a, b, h, g) - r0q) * (2 * kD) + 16 * t16;  // bytes from head row 0
      lds_dma16(buffer_rsrc(a.q + r0q * kD, INT_MAX), lds_ptr(s_r4) + h * (kWaveChunks * 16), dq);  // rows of later queries lie Hq rows on
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }

    // ---- rotated queries H (s * q): lane (g = q4, j = t16) holds coordinates 8 j .. 8 j + 7 ----
    float qmax_l;
    {
      float x[8];
      const uint4 raw = *reinterpret_cast<const uint4*>(qreg + 16 * lane);
      const uint32_t qw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = half_bits_to_float(qw[i] & 0xffffu);
        x[2 * i + 1] = half_bits_to_float(qw[i] >> 16);
      }
      const int j = t16;
      const uint32_t swd = j < 4 ? a.signs.w[0] : j < 8 ? a.signs.w[1] : j < 12 ? a.signs.w[2] : a.signs.w[3];
      const uint32_t sb = (swd >> (8 * (j & 3))) & 0xffu;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((sb >> e) & 1u) x[e] = -x[e];
      wht_row8_dpp<16>(x, j);
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[e]));
      qmax_l = max16(mx) * a.qscale;
      // rotated rows as fp32 [4][128] over the raw rows (this wave's region; LDS keeps its order)
      float4* d = reinterpret_cast<float4*>(qreg + 512 * q4 + 32 * j);
      d[0] = make_float4(x[0], x[1], x[2], x[3]);
      d[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    // scale exponent of head g: its largest |q| * qscale lands near 2^13
    const float qm0 = lane_value(qmax_l, 0), qm1 = lane_value(qmax_l, 16);
    const float qm2 = lane_value(qmax_l, 32), qm3 = lane_value(qmax_l, 48);
    auto head_exp = [&](int g) {
      const float qm = g == 0 ? qm0 : g == 1 ? qm1 : g == 2 ? qm2 : qm3;
      return qm > 0.0f ? 13 - ilogbf(qm) : 0;
    };

    // QK A operand, step mi: row t16 = (query head t16 >> 2, fp16 part t16 & 1; rows with
    // (t16 >> 1) & 1 are zero); K holds the coordinates of code bytes 2 mi, 2 mi + 1 of this
    // lane's word order, [x_a, x_b, x_a, x_b, x_c, x_d, x_c, x_d] against the centroid parts
    // [hi, hi, lo, lo, hi, hi, lo, lo].
    uint4 aq[8];
    {
      const int g = t16 >> 2;
      const bool live = ((t16 >> 1) & 1) == 0 && g < G;
      const bool lo_part = t16 & 1;
      const float f = live ? ldexpf(a.qscale, head_exp(g)) : 0.0f;
      // this lane's 32 coordinates 32 q4 .. 32 q4 + 31 in word order (upper 16 first if sw)
      const uint8_t* src = qreg + 512 * (live ? g : 0);
      float x[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c4 = (i + 4 * sw) & 7;  // 4-coordinate group at word-order position i
        const float4 v = *reinterpret_cast<const float4*>(src + 128 * q4 + 16 * c4);
        x[4 * i] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
      }
#pragma unroll
      for (int mi = 0; mi < 8; ++mi) {
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t hi, lo;
          split_half(live ? x[4 * mi + i] * f : 0.0f, hi, lo);
          p[i] = lo_part ? lo : hi;
        }
        const uint32_t ab = p[0] | (p[1] << 16), cd = p[2] | (p[3] << 16);
        aq[mi] = make_uint4(ab, ab, cd, cd);
      }
    }
    // softmax lane: token t16, query head g0 = q4
    const int g0 = q4;
    const bool live0 = g0 < G;
    const float f0 = live0 ? ldexpf(1.0f, -(head_exp(g0) + kLutShift)) : 0.0f;
    const int lim0 = min(u.end, u.seq_len - a.nq + a.q0 + g0 / a.g_real + 1);  // causal limit of head g0
    const int lo_l = u.ns - t16;                                              // p >= ns
    const int hi_l = live0 ? lim0 - t16 : INT_MIN;                            // p < lim0

    float m_s = kSent, m_w = kSent, l_s = 0.0f;
    float t_s = kSent + kThr, t_w = kSent + kThr, m_b = kSent - (float)kWShift;  // thresholds, weight base
    float4_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- key half of one run: table entries of this lane's 16 code bytes, and the norms ----
    auto key_codes = [&](const uint8_t* buf, uint32_t (&w)[4], float& kn, float& vn) {
      const u32x2 r0 = *reinterpret_cast<const u32x2*>(at(buf, off_k0));
      const u32x2 r1 = *reinterpret_cast<const u32x2*>(at(buf, off_k1));
      kn = *reinterpret_cast<const float*>(at(buf, off_kn));
      vn = *reinterpret_cast<const float*>(at(buf, off_vn));
      w[0] = r0.x;
      w[1] = r0.y;
      w[2] = r1.x;
      w[3] = r1.y;
    };
    auto key_lookup = [&](const uint32_t (&w)[4], uint2 (&ke)[16]) {
#pragma unroll
      for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t byte = 2 * (mi & 1) + j;
          const uint32_t off = __builtin_amdgcn_perm(w[mi >> 1], kcopy, 0x0c0c0000u | ((4u + byte) << 8));
          ke[2 * mi + j] = *reinterpret_cast<const uint2*>(tab + off);
        }
      }
    };
    // QK: this lane's score (token t16, head g0) before the norm and scales
    auto key_mfma = [&](const uint2 (&ke)[16]) {
      float4_t sa = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        sa = mfma16(aq[mi], make_uint4(ke[2 * mi].x, ke[2 * mi].y, ke[2 * mi + 1].x, ke[2 * mi + 1].y), sa);
      return sa[0] + sa[1];
    };

    // value entries of one run: tokens (q4, q4 + 4) then (q4 + 8, q4 + 12), code byte mi of dword t16
    auto value_lookup = [&](const uint32_t (&cw)[4], uint2 (&ve)[16]) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const uint32_t sel = 0x0c0c0000u | ((4u + mi) << 8);
          ve[8 * hf + 2 * mi] = *reinterpret_cast<const uint2*>(tab + __builtin_amdgcn_perm(cw[2 * hf], kcopy, sel));
          ve[8 * hf + 2 * mi + 1] =
              *reinterpret_cast<const uint2*>(tab + __builtin_amdgcn_perm(cw[2 * hf + 1], kcopy, sel));
        }
      }
    };
    auto value_codes = [&](const uint8_t* buf, uint32_t (&cw)[4]) {
#pragma unroll
      for (int m = 0; m < 4; ++m) cw[m] = *reinterpret_cast<const uint32_t*>(at(buf, off_v[m]));
    };

    // Pipeline state carried from step s - 1: run s's raw scores and norms (token t16) and its value
    // entries.  Step s issues run s + 1's key lookups, then does run s's softmax and PV, then
    // issues run s + 1's value lookups (after PV has consumed run s's) and does run s + 1's QK.
    // Table lookups stay in flight across the step barrier; every read of a run buffer is
    // consumed within its step, before the barrier that can release the buffer.
    float sc = 0.0f, knf = 0.0f, lv = 0.0f;  // run s: raw score, n_K * f0, log2 n_V (token t16)
    uint2 ve[16];
    auto body = [&](int s, const uint8_t* nxt) {
      uint32_t kw[4], cw[4];
      float kn1, vn1;
      key_codes(nxt, kw, kn1, vn1);
      value_codes(nxt, cw);
      __builtin_amdgcn_sched_barrier(0);  // the code reads go out first
      uint2 ke[16];
      key_lookup(kw, ke);

      // softmax of run s, lane (token t16, head g0); masked rows never touch their garbage norms.
      // The references m_s (scores) and m_w (scores + log2 n_V) move only when some score passes
      // them by more than kThr: terms stay below 2^kThr, weights below 2^(kWShift + kThr).
      const int pb = (run0 + s) * 16;
      const bool valid = pb >= lo_l && pb < hi_l;
      const float s0 = valid ? sc * knf : -INFINITY;
      const float sw0 = valid ? s0 + lv : -INFINITY;  // + log2(n_V)
      if (__builtin_amdgcn_ballot_w64(s0 > t_s || sw0 > t_w) != 0) {
        const float ns2 = fmaxf(m_s, max16(s0)), nw2 = fmaxf(m_w, max16(sw0));
        l_s *= __builtin_amdgcn_exp2f(m_s - ns2);
        const float r = __builtin_amdgcn_exp2f(m_w - nw2);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] *= r;
        m_s = ns2;
        m_w = nw2;
        t_s = m_s + kThr;
        t_w = m_w + kThr;
        m_b = m_w - (float)kWShift;
      }
      l_s += __builtin_amdgcn_exp2f(s0 - m_s);
      const float wt = __builtin_amdgcn_exp2f(sw0 - m_b);
      const auto h2 = __builtin_amdgcn_cvt_pkrtz(wt, 0.0f);
      const auto p2 = __builtin_amdgcn_cvt_pkrtz(wt, wt - (float)h2[0]);
      const uint32_t wpk = __builtin_bit_cast(uint32_t, p2);  // both fp16 parts of the weight

      // PV A operands: tokens q4 + 4 m of head t16 >> 2, one weight part, at the row's nibble
      uint32_t wg[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) wg[m] = __builtin_amdgcn_ds_bpermute(bp_base + 16 * m, wpk);
      uint32_t d[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) d[m] = __builtin_amdgcn_perm(wg[m], wg[m], bp_sel);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint4 aw = make_uint4(d[2 * hf], d[2 * hf], d[2 * hf + 1], d[2 * hf + 1]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const uint2 e0 = ve[8 * hf + 2 * mi], e1 = ve[8 * hf + 2 * mi + 1];
          acc[mi] = mfma16(aw, make_uint4(e0.x, e0.y, e1.x, e1.y), acc[mi]);
        }
      }
      value_lookup(cw, ve);  // run s + 1
      sc = key_mfma(ke);
      // the norms of run s + 1 are used here, so no read of its buffer outlives the step
      knf = kn1 * f0;
      lv = __builtin_amdgcn_logf(vn1);
    };

    if (n_run > 0) {
      lds_barrier();  // run 0 is in
      {
        uint32_t kw[4], cw[4];
        uint2 ke[16];
        float kn0, vn0;
        key_codes(s_r0, kw, kn0, vn0);
        value_codes(s_r0, cw);
        key_lookup(kw, ke);
        value_lookup(cw, ve);
        sc = key_mfma(ke);
        knf = kn0 * f0;
        lv = __builtin_amdgcn_logf(vn0);
      }
      // step s: barrier (run s + 1 is in; run s's buffer, read and used up by step s - 1, may be
      // refilled), then the body.  After the last run the body reads a buffer that holds no run;
      // its results are unused.
      for (int s = 0; s < n_run; s += kRing) {
        step_barrier();
        body(s, s_r1);
        if (s + 1 < n_run) {
          step_barrier();
          body(s + 1, s_r2);
        }
        if (s + 2 < n_run) {
          step_barrier();
          body(s + 2, s_r3);
        }
        if (s + 3 < n_run) {
          step_barrier();
          body(s + 3, s_r4);
        }
        if (s + 4 < n_run) {
          step_barrier();
          body(s + 4, s_r0);
        }
      }
    }

    // ---- this wave's partial for head g0: coordinates 8 t16 + 2 mi + nibble ----
    l_s += dpp<kDppQuadXor1>(l_s);
    l_s += dpp<kDppQuadXor2>(l_s);
    l_s += dpp<kDppHalfRowMirror>(l_s);
    l_s += dpp<kDppRowMirror>(l_s);
    if (live0) {
      const float c0 = __builtin_amdgcn_exp2f(m_w - m_s) * ldexpf(1.0f, -(kWShift + kLutShift));
      float* part = a.partials + ((((int64_t)b * kH + h) * a.part_stride + u.split) * G + g0) * (kD + 2);
      float2* o = reinterpret_cast<float2*>(part + 2 + 8 * t16);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        o[mi] = make_float2((acc[mi][0] + acc[mi][1]) * c0, (acc[mi][2] + acc[mi][3]) * c0);
      if (t16 == 0) *reinterpret_cast<float2*>(part) = make_float2(m_s, l_s);
    }
  }
}

}  // namespace

// Whether the block-streaming kernel serves a format: K4/V4 at D = 128, eight kv heads, unpadded
// plain slots (norm correction changes the stored norm only), one codebook array for keys and
// values, page blocks of whole 16-position runs, at most four query heads per kv head.
bool tq_decode_block_format(const TqLayer& L) {
  return L.D == 128 && L.kb == 4 && L.vb == 4 && L.Hkv == kH && L.stride == kSB && L.slot_bytes == kSB &&
         !L.mean && !L.qjl && L.bs % 16 == 0 && L.G <= 4 && L.kc == L.vc;
}

// Split geometry of the block kernel: about one (sequence, split) unit per compute unit, splits of
// whole runs, at most kMaxRuns runs each.
TqSplit tq_decode_block_split(int num_seqs, int max_seq_len) {
  constexpr long kUnits = 256;  // compute units of the MI355X
  const long tokens = max_seq_len > 0 ? max_seq_len : 1;
  long chunk = (tokens * num_seqs + kUnits - 1) / kUnits;
  chunk = ((chunk + 15) / 16) * 16;
  if (chunk < 64) chunk = 64;
  if (chunk > 16L * kMaxRuns) chunk = 16L * kMaxRuns;
  TqSplit sp;
  sp.chunk = (int)chunk;
  sp.max_split = (int)((tokens + chunk - 1) / chunk);
  return sp;
}

int tq_launch_decode_block(const TqLayer& L, const void* q, const void* pages, const int32_t* block_tables,
                           int max_blocks, const int32_t* seq_lens, int num_seqs, const TqSplit& sp,
                           int n_sink, const int32_t* win_lens, int win_cap, float qscale, float* partials,
                           int part_stride, int nq, int q0, int g_real, void* stream) {
  if (sp.chunk % 16 != 0 || sp.chunk > 16 * kMaxRuns) return (int)hipErrorInvalidValue;
  TqBlockArgs a;
  a.q = (const uint16_t*)q;
  a.pages = (const uint8_t*)pages;
  a.bt = block_tables;
  a.seq_lens = seq_lens;
  a.win_lens = win_cap > 0 ? win_lens : nullptr;
  a.partials = partials;
  a.c = L.kc;
  a.signs = L.signs;
  a.qscale = qscale;
  a.max_blocks = max_blocks;
  a.bs = L.bs;
  a.bs_shift = -1;
  for (int s = 0; s < 31; ++s)
    if ((1 << s) == L.bs) a.bs_shift = s;
  a.G = L.G;
  a.Hq = L.Hq;
  a.n_sink = n_sink;
  a.win_cap = win_cap;
  a.chunk = sp.chunk;
  a.max_split = sp.max_split;
  a.part_stride = part_stride;
  a.n_units = num_seqs * sp.max_split;
  a.nq = nq;
  a.q0 = q0;
  a.g_real = g_real;
  const int grid = a.n_units < 256 ? a.n_units : 256;
  hipLaunchKernelGGL(tq_decode_block_kernel, dim3(grid), dim3(kT + 256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}
