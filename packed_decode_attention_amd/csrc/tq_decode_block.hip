// Fused paged decode attention over packed TQ pages, whole-block streaming kernel (gfx950), for
// page formats at D = 128 with eight kv heads of unpadded slots: K4/V4 with one codebook for keys
// and values and up to four query heads per kv head (the Llama-3-8B-shaped workload), and K3/V2
// with up to eight (the ragged serving batch).
//
// Method as in tq_decode.hip: scores on the codes with a rotated query, online softmax, values
// summed in the rotated frame, split-K partials merged by tq_decode_merge_kernel (tq-kv, "Custom
// CUDA Kernel Stack": split-KV flash decode on compressed KV; turboquant-pro 1.4.2, "Fused CUDA
// decode": split-K decode on the codes).  What differs is how page bytes reach the matrix cores:
//  * One persistent workgroup of 12 waves per compute unit: compute wave h (0..7) computes kv
//    head h, and four producer waves issue every page load.  The workgroup reads whole page runs
//    (16 positions x 8 heads, contiguous: 17 KB at K4/V4, 11 KB at K3/V2): each load instruction
//    moves 1 KB of page bytes straight into LDS (buffer_load ... lds), in a ring of five run
//    buffers (four in flight while one is read).  The compute waves issue no vector memory
//    instruction inside the run loop.  Fetching one kv head's rows instead (136 bytes every 1088
//    at K4/V4) streams about a quarter slower on this chip.
//  * Balanced work: the runs of all sequences form one sequence, and workgroup k takes the k-th
//    contiguous range of it, so a ragged batch gives every compute unit the same number of runs.
//    A range splits into pieces at sequence boundaries; each piece writes one partial, and
//    workgroup 0 records each sequence's piece count for the merge.
//  * LDS reads are free of bank conflicts.  The loads place the 16-byte chunks of a run rotated
//    by (position / 4) within each aligned group of 16 chunks (the loads choose their source
//    chunks, the LDS side stays contiguous), so the 16 positions of a run, a page row apart, no
//    longer fall on 4 banks.  The centroid operand tables (one code group -> fp16 high and low
//    parts of its two centroids, 8 bytes: a byte of 4-bit codes, six bits of 3-bit codes, a
//    nibble of 2-bit codes) are held in 32 interleaved copies, lane l reading copy l mod 32: the
//    32 lanes of each LDS pass read distinct bank pairs.
//  * QK on v_mfma_f32_16x16x32_f16: rows are (query head, fp16 part of the query), columns the 16
//    positions, K the coordinates with both fp16 parts of each centroid.  PV: rows are (query
//    head, fp16 part of the weight, which coordinate of the code group), columns the code groups
//    a lane holds (two coordinates each), K the positions with both centroid parts; every row is
//    live, and the code group of one position indexes the table directly.  With eight query
//    heads per kv head the QK rows are all live and PV takes two row sets.
//  * Software pipeline: each step issues the next run's key lookups, then does the current run's
//    softmax and PV, then the next run's QK.  The running maxima are rescaled lazily (only when a
//    run's maximum exceeds the reference by more than two, in log2 units), which keeps the step
//    one basic block in the common case.

#include <climits>

#include "../../include/tq.h"
#include "tq_quant_device.h"

namespace {
using namespace tqd;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // one 8-byte LDS read

constexpr int kW = 8;                          // compute waves per workgroup: one per kv head
constexpr int kT = kW * 64;                    // compute threads
constexpr int kNP = 4;                         // producer waves
constexpr int kThreads = kT + 64 * kNP;        // threads per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kH = 8;                          // kv heads
constexpr int kD = 128;
constexpr int kRing = 5;                       // run buffers
constexpr int kCP = 32;                        // table copies
constexpr int kLutShift = 8;                   // table entries hold c * 2^8
constexpr int kWShift = 13;                    // weights enter PV as w * 2^13 (below 2^15)
constexpr float kThr = 2.0f;                   // lazy rescale threshold, log2 units
constexpr float kSent = -1.0e30f;              // finite minus infinity of the running maxima
constexpr int kMaxRuns = 1024;                 // runs per unit (sixteen lanes' worth of run rows)
constexpr int kPlanInts = 48;                  // LDS words of the work plan (3 per wave, 8 more)
constexpr int kGrid = 256;                     // workgroups: one per compute unit of the MI355X

// Geometry of one page format: KB-bit keys, VB-bit values, up to GM query heads per kv head.
template <int KB, int VB, int GM>
struct Fmt {
  static constexpr int kKCode = kD * KB / 8;         // K code bytes (the K norm follows)
  static constexpr int kVOff = kKCode + 4;           // V region offset in a slot
  static constexpr int kVCode = kD * VB / 8;
  static constexpr int kSB = kVOff + kVCode + 4;     // slot bytes: 136 at K4/V4, 88 at K3/V2
  static constexpr int kRowBytes = kH * kSB;         // one position, every kv head
  static constexpr int kRunBytes = 16 * kRowBytes;   // one run of 16 positions
  static constexpr int kLoads = kRunBytes / 1024;    // 1 KB loads per run
  static constexpr int kLoadsHi = (kLoads + kNP - 1) / kNP;  // loads per run of producer p <
  static constexpr int kLoadsLo = kLoads / kNP;              // kLoads % kNP, and of the others
  static constexpr int kGroupChunks = kRowBytes / 4;  // 16-byte chunks of four positions
  static constexpr bool kOneTable = KB == VB;        // K and V share the table (one codebook)
  static constexpr int kKEnt = KB == 4 ? 256 : 64;   // K table entries: a byte, or six bits
  static constexpr int kVEnt = kOneTable ? 0 : (VB == 4 ? 256 : 16);
  static constexpr int kVTab = kOneTable ? 0 : kKEnt * 256;  // V table byte offset
  static constexpr int kBuf0 = (kKEnt + kVEnt) * 256;        // first run buffer, after the tables
  static constexpr int kNZ = GM / 4;                 // query heads per softmax lane
  // The queries of a piece's first unit are staged in the last run buffer when a wave's share of
  // it holds GM fp32 rows (the buffer takes a run only after the first step); else in a region of
  // their own after the ring.
  static constexpr int kQBytes = GM * 512;           // per wave: GM rotated fp32 rows
  static constexpr bool kQInRing = kRunBytes / kW >= kQBytes;
  static constexpr int kQBase = kBuf0 + kRing * kRunBytes;
  static constexpr int kPlanOff = kQBase + (kQInRing ? 0 : kW * kQBytes);
  static constexpr int kLdsBytes = kPlanOff + 4 * kPlanInts;
  static_assert(kRunBytes % 1024 == 0, "runs are whole 1 KB loads");
  static_assert(kRowBytes % 64 == 0, "four positions are whole groups of 16 chunks");
  static_assert(kLoadsHi <= 5 && kLoadsHi * 3 <= 63, "source offsets and wait counts");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

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

__device__ __forceinline__ float sum16(float x) {  // sum over a 16-lane row, in every lane
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppHalfRowMirror>(x);
  return x + dpp<kDppRowMirror>(x);
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

// LDS placement of a run: byte g of the run (position g / row bytes) sits in chunk slot
// ((g / 16 + q) mod 16) of its aligned group of 16 chunks, q = the position divided by four
// (QC = chunks of four positions).  A group never straddles two values of q.
template <int QC>
__device__ __forceinline__ int run_lds_offset(int g) {
  const int c = g >> 4, q = c / QC;
  return (((c & ~15) | ((c + q) & 15)) << 4) | (g & 15);
}
// The run chunk that LDS chunk p holds (the inverse of the placement above).
template <int QC>
__device__ __forceinline__ int run_chunk_at(int p) {
  const int q = p / QC;
  return (p & ~15) | ((p - q) & 15);
}

// Inclusive prefix sum and maximum across a wave (the work plan only), by DPP: row shifts within
// each 16-lane row, then row broadcasts of lanes 15 and 31 into the later rows.  Lanes a step has
// no source for add 0 (counts are non-negative, so 0 also serves the maximum).
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_int(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_int<0x111>(x);        // row_shr:1
  x += dpp_int<0x112>(x);        // row_shr:2
  x += dpp_int<0x114>(x);        // row_shr:4
  x += dpp_int<0x118>(x);        // row_shr:8
  x += dpp_int<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_int<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ int wave_incl_max(int x) {
  x = max(x, dpp_int<0x111>(x));
  x = max(x, dpp_int<0x112>(x));
  x = max(x, dpp_int<0x114>(x));
  x = max(x, dpp_int<0x118>(x));
  x = max(x, dpp_int<0x142, 0xa>(x));
  x = max(x, dpp_int<0x143, 0xc>(x));
  return x;
}
// Sum and maximum over the wave (lane 63 of the inclusive forms), wave-uniform.
__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_incl_scan(x), 63); }
__device__ __forceinline__ int wave_max(int x) { return __builtin_amdgcn_readlane(wave_incl_max(x), 63); }

}  // namespace

struct TqBlockArgs {
  const uint16_t* q;
  const uint8_t* pages;
  const int32_t* bt;
  const int32_t* seq_lens;
  const int32_t* win_lens;  // NULL: no hot window
  float* partials;          // [B][8][part_stride][G][D + 2]
  int32_t* nsplit;          // [B]: pieces (partials) of each sequence, written by workgroup 0
  const float* kc;          // key codebook (2^KB centroids)
  const float* vc;          // value codebook (2^VB centroids)
  TqSigns signs;
  float qscale;             // scale * log2(e) / sqrt(D)
  int max_blocks, bs, bs_shift, G, Hq, n_sink, win_cap;
  int num_seqs, part_stride, max_pieces, max_parts, max_runs;
  int nq, q0, g_real;       // several queries per sequence (one: 1, 0, G)
  // Fused append (k_new NULL: none).  The new token of each sequence, K and V rows [B][8][128]
  // fp16, is quantized into the page slot of position seq_len - 1 by the workgroup whose share
  // holds that position's run, before that workgroup loads any run.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* pages_w;         // the pages, written
  const float* kt;          // key boundaries (2^KB - 1)
  const float* vt;          // value boundaries
  float rsqrt_d;            // 1 / sqrt(D)
};

// Sequences whose new token one workgroup quantizes at most (the host bounds the batch by it),
// and the fused append's scratch in the last run buffer: boundaries [2][256] floats, the K and V
// bucket tables, their shifts, the list of sequences.
constexpr int kAppendMax = TQ_APPEND_MAX_SEQS;
constexpr int kAppTabOff = 2048;
constexpr int kAppShOff = kAppTabOff + 2 * 130 * 8;
constexpr int kAppListOff = kAppShOff + 64;

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

// The packed positions of a sequence, [ns, end), read as runs run0 .. run0 + n_run - 1 (the run
// holding ns first; rows below ns and from end on are masked).  Sinks and hot-window rows come
// from the fp16-row chunks.
struct TqSeq {
  int seq_len, ns, end, run0, n_run;
};

template <bool UNIFORM>
__device__ __forceinline__ TqSeq seq_of(const TqBlockArgs& a, int b) {
  TqSeq s;
  s.seq_len = UNIFORM ? load_uniform(a.seq_lens + b) : a.seq_lens[b];
  s.ns = min(a.n_sink, s.seq_len);
  int win = 0;
  if (a.win_lens != nullptr) {
    const int wl = UNIFORM ? load_uniform(a.win_lens + b) : a.win_lens[b];
    win = max(0, min(wl, min(a.win_cap, s.seq_len - s.ns)));
  }
  s.end = s.seq_len - win;
  s.run0 = s.ns >> 4;
  s.n_run = s.end > s.ns ? ((s.end - 1) >> 4) - s.run0 + 1 : 0;
  return s;
}

// A sequence record in five LDS words.
__device__ __forceinline__ void put_seq(int* w, const TqSeq& s) {
  w[0] = s.seq_len;
  w[1] = s.ns;
  w[2] = s.end;
  w[3] = s.run0;
  w[4] = s.n_run;
}
__device__ __forceinline__ TqSeq get_seq(const int* w) { return TqSeq{w[0], w[1], w[2], w[3], w[4]}; }

// This workgroup's share of the batch, in one of two forms.
//  * Aligned: when the sequences with packed runs split evenly over the workgroups (c of them per
//    sequence, no piece longer than an even share of all runs), workgroup k takes piece k mod c of
//    the (k / c)-th such sequence, and no workgroup switches sequences.
//  * Ranges: otherwise the sequences with runs are laid end to end on one cost axis, each as
//    kTqUnitCostRuns of fixed cost followed by its runs, and workgroup k takes the runs in cost
//    [S, E), rpw per workgroup, cut into pieces at sequence boundaries; b is the first sequence
//    in the share and R the cost position of its run 0.  A workgroup pays the fixed cost of every
//    unit it starts (its queries, block-table rows and first runs arrive before it can compute),
//    so one that touches many short sequences takes fewer runs.
// A piece is cut into units of at most kMaxRuns runs, and every unit writes a partial of its own:
// a sequence's partials are numbered in run order, part0 being that of the share's first unit.
// Workgroup 0 writes each sequence's partial count.  Every thread of the workgroup calls it.  An
// aligned piece is walked as a share of one sequence whose runs count from its first run (R = 0).
// The host bounds the batch's runs by INT32_MAX, so 32-bit counts suffice.
struct TqPlan {
  int S, E, R, rpw, b, part0;
  TqSeq sq0;  // sequence b
};

constexpr int kAlignSlack = 2;  // runs an aligned piece may exceed the even share by

__device__ __forceinline__ int units_of(int runs) { return (runs + kMaxRuns - 1) / kMaxRuns; }

// Units of share k (runs [k rpw, (k + 1) rpw)) inside a sequence's runs [R, R + n).
__device__ __forceinline__ int units_in_share(int k, int rpw, int R, int n) {
  const int64_t lo = max((int64_t)k * rpw, (int64_t)R), hi = min((int64_t)(k + 1) * rpw, (int64_t)R + n);
  return hi > lo ? units_of((int)(hi - lo)) : 0;
}

// n_own: the run count of sequence tid (0 past the batch), loaded by the caller at kernel entry so
// the load overlaps the table fill.  A batch of at most kThreads sequences takes one pass over
// the run counts; a larger one takes a second, kThreads sequences at a time.
__device__ TqPlan make_plan(const TqBlockArgs& a, int* s_plan, int* s_list, int tid, int wave, int lane,
                           const TqSeq& own) {
  const int n_own = own.n_run;
  const int B = a.num_seqs;
  const bool one_pass = B <= kThreads;
  // total runs, sequences with runs, longest sequence (and, in one pass, the prefixes)
  int t = 0, nz = 0, mx = 0, incl = 0, incl_nz = 0;
  if (one_pass) {
    incl = wave_incl_scan(n_own);
    incl_nz = wave_incl_scan(n_own > 0);
    t = __builtin_amdgcn_readlane(incl, 63);
    nz = __builtin_amdgcn_readlane(incl_nz, 63);
    mx = n_own;
  } else {
    for (int b = tid; b < B; b += kThreads) {
      const int n = seq_of<false>(a, b).n_run;
      t += n;
      nz += n > 0;
      mx = max(mx, n);
    }
    t = wave_sum(t);
    nz = wave_sum(nz);
  }
  mx = wave_max(mx);
  if (lane == 0) {
    s_plan[wave] = t;
    s_plan[kWaves + wave] = nz;
    s_plan[2 * kWaves + wave] = mx;
  }
  if (tid == 0) {
    s_plan[3 * kWaves] = -1;
    s_plan[3 * kWaves + 7] = 0;  // fused append: sequences in s_list
  }
  __syncthreads();
  // the waves' totals, lane w holding wave w's, reduced across the wave
  const int st = wave_incl_scan(lane < kWaves ? s_plan[lane] : 0);
  const int sz = wave_incl_scan(lane < kWaves ? s_plan[kWaves + lane] : 0);
  const int T = __builtin_amdgcn_readlane(st, 63), NZS = __builtin_amdgcn_readlane(sz, 63);
  const int MX = wave_max(lane < kWaves ? s_plan[2 * kWaves + lane] : 0);
  const int base = wave > 0 ? __builtin_amdgcn_readlane(st, wave - 1) : 0;
  const int base_nz = wave > 0 ? __builtin_amdgcn_readlane(sz, wave - 1) : 0;
  // runs per workgroup: an even share, and enough that no sequence (at most max_runs runs) spans
  // more than max_pieces - 1 workgroups ((n - 1) / rpw + 2 at most); the ranges take an even share
  // of the cost axis (runs plus kTqUnitCostRuns per sequence with runs; the host bounds it by
  // INT32_MAX), with the same floor
  const int floor_rpw = (int)(((int64_t)a.max_runs + a.max_pieces - 3) / (a.max_pieces - 2));
  int rpw = (int)(((int64_t)T + gridDim.x - 1) / gridDim.x);
  if (rpw < floor_rpw) rpw = floor_rpw;
  if (rpw < 1) rpw = 1;
  const int TC = T + kTqUnitCostRuns * NZS;  // length of the cost axis
  int cpw = (int)(((int64_t)TC + gridDim.x - 1) / gridDim.x);
  if (cpw < floor_rpw) cpw = floor_rpw;
  if (cpw < 1) cpw = 1;
  const int c = NZS > 0 ? min((int)gridDim.x / NZS, a.max_pieces - 1) : 0;  // aligned pieces per sequence
  const bool aligned = c >= 1 && (MX + c - 1) / c <= rpw + kAlignSlack;
  const int k = blockIdx.x;
  TqPlan p;
  p.rpw = cpw;
  p.S = (int)min((int64_t)k * cpw, (int64_t)TC);
  p.E = min(p.S + cpw, TC);
  p.b = B;
  p.R = p.E;
  p.part0 = 0;
  const int target = c > 0 ? k / c : 0;  // aligned: the target-th sequence with runs
  // sequence b with n runs, the runs before it and its rank among the sequences with runs: the
  // partial count for the merge, and whether this workgroup's share starts in it
  auto place = [&](int b, const TqSeq& sq, int before, int rank) {
    const int n = sq.n_run;
    const int R = before + kTqUnitCostRuns * (rank + 1);  // cost position of its run 0
    int parts = 0;
    if (n > 0) {
      if (aligned) {
        const int ps = (n + c - 1) / c;  // runs per aligned piece of this sequence
        const int pieces = (n + ps - 1) / ps;
        parts = (pieces - 1) * units_of(ps) + units_of(n - (pieces - 1) * ps);
        if (rank == target) {
          s_plan[3 * kWaves] = b;
          s_plan[3 * kWaves + 1] = ps;
          put_seq(s_plan + 3 * kWaves + 2, sq);
        }
      } else {
        for (int kk = R / cpw; kk <= (R + n - 1) / cpw; ++kk) parts += units_in_share(kk, cpw, R, n);
        if (R - kTqUnitCostRuns <= p.S && p.S < R + n) {  // from its fixed cost to its last run
          s_plan[3 * kWaves] = b;
          s_plan[3 * kWaves + 1] = R;
          put_seq(s_plan + 3 * kWaves + 2, sq);
        }
      }
    }
    // (a sequence longer than the host's bound would have more partials than slots: those past
    // the bound are neither computed nor merged)
    if (k == 0) a.nsplit[b] = min(parts, a.max_parts);
    // fused append: the workgroup holding the last run (the new token's) lists the sequence
    if (a.k_new != nullptr && n > 0) {
      const int owner = aligned ? rank * c + (n - 1) / ((n + c - 1) / c) : (R + n - 1) / cpw;
      if (owner == k) {
        const int i = atomicAdd(&s_plan[3 * kWaves + 7], 1);
        if (i < kAppendMax) s_list[i] = b;
      }
    }
  };
  if (one_pass) {
    if (tid < B) place(tid, own, base + incl - n_own, base_nz + incl_nz - 1);
  } else {
    __syncthreads();
    // exclusive prefixes of the run counts and of the sequences with runs, kThreads at a time
    int carry = 0, carry_nz = 0;
    for (int c0 = 0; c0 < B; c0 += kThreads) {
      const int b = c0 + tid;
      TqSeq sq{};
      if (b < B) sq = seq_of<false>(a, b);
      const int n = sq.n_run;
      const int in = wave_incl_scan(n);
      const int in_nz = wave_incl_scan(n > 0);
      if (lane == 63) {
        s_plan[wave] = in;
        s_plan[kWaves + wave] = in_nz;
      }
      __syncthreads();
      const int ct = wave_incl_scan(lane < kWaves ? s_plan[lane] : 0);
      const int cz = wave_incl_scan(lane < kWaves ? s_plan[kWaves + lane] : 0);
      const int total = __builtin_amdgcn_readlane(ct, 63), total_nz = __builtin_amdgcn_readlane(cz, 63);
      const int bs = carry + (wave > 0 ? __builtin_amdgcn_readlane(ct, wave - 1) : 0);
      const int bs_nz = carry_nz + (wave > 0 ? __builtin_amdgcn_readlane(cz, wave - 1) : 0);
      if (b < B) place(b, sq, bs + in - n, bs_nz + in_nz - 1);
      carry += total;
      carry_nz += total_nz;
      __syncthreads();
    }
  }
  __syncthreads();
  const int found = s_plan[3 * kWaves];
  p.sq0 = TqSeq{};
  if (found >= 0) {
    const int f1 = s_plan[3 * kWaves + 1];
    p.sq0 = get_seq(s_plan + 3 * kWaves + 2);
    const int n = p.sq0.n_run;
    p.b = found;
    if (aligned) {  // piece j of the sequence, runs [j ps, (j + 1) ps)
      const int j = k - target * c, ps = f1;
      p.R = 0;
      p.S = min(n, j * ps);
      p.E = min(n, j * ps + ps);
      p.rpw = INT_MAX;
      p.part0 = j * units_of(ps);
    } else {  // units of the earlier shares in the first sequence
      p.R = f1;
      for (int kk = f1 / cpw; kk < k; ++kk) p.part0 += units_in_share(kk, cpw, f1, n);
    }
  }
  // The values are the same in every lane (LDS reads and cross-lane sums the compiler cannot
  // prove uniform): in scalar registers the unit loops branch on scalars.
  p.S = __builtin_amdgcn_readfirstlane(p.S);
  p.E = __builtin_amdgcn_readfirstlane(p.E);
  p.R = __builtin_amdgcn_readfirstlane(p.R);
  p.rpw = __builtin_amdgcn_readfirstlane(p.rpw);
  p.b = __builtin_amdgcn_readfirstlane(p.b);
  p.part0 = __builtin_amdgcn_readfirstlane(p.part0);
  p.sq0.seq_len = __builtin_amdgcn_readfirstlane(p.sq0.seq_len);
  p.sq0.ns = __builtin_amdgcn_readfirstlane(p.sq0.ns);
  p.sq0.end = __builtin_amdgcn_readfirstlane(p.sq0.end);
  p.sq0.run0 = __builtin_amdgcn_readfirstlane(p.sq0.run0);
  p.sq0.n_run = __builtin_amdgcn_readfirstlane(p.sq0.n_run);
  return p;
}

// The units of a plan in order: f(seq, b, run_first, n_run, part) is called in the same order,
// with the same wave-uniform values, in every wave.
template <typename Fn>
__device__ __forceinline__ void for_each_unit(const TqBlockArgs& a, const TqPlan& p, Fn&& f) {
  int R = p.R, part = p.part0;
  for (int b = p.b; R < p.E && b < a.num_seqs; ++b) {
    const TqSeq sq = b == p.b ? p.sq0 : seq_of<true>(a, b);
    const int hi = min(p.E, R + sq.n_run);
    for (int u0 = max(p.S, R); u0 < hi && part < a.max_parts; u0 += kMaxRuns, ++part)
      f(sq, b, sq.run0 + (u0 - R), min(kMaxRuns, hi - u0), part);
    R += sq.n_run + (sq.n_run > 0 ? kTqUnitCostRuns : 0);  // run 0 of the next sequence
    part = 0;  // a later sequence starts in this share
  }
}

// Destination of the fused append's stores for rows past the listed tokens (a tile's lanes all
// store).
__device__ __align__(16) uint8_t tq_block_append_discard[256];

// Fused append: the new tokens of the n_list sequences in s_list (their last runs are this
// workgroup's), quantized exactly as tq_quantize_kernel does (the same region code, Hadamard
// operands and bucket tables) into the slots of their positions seq_len - 1, before the workgroup
// loads any run that holds one.  Scratch in `region` (the last run buffer, which takes a run only
// after the first unit's first step): boundaries, tables, table shifts.  tk, tv: boundary j of K
// and V in lane j of wave 0.  Every thread calls it, at the same point of the first unit; its
// barriers leave the producers' run loads in flight, and the compute waves' stores are complete
// at the last one.
template <int KB, int VB>
__device__ __forceinline__ void append_tokens(const TqBlockArgs& a, uint8_t* region, const int* s_list,
                                              int n_list, int tid, int wave, int lane, float tk, float tv) {
  using F = Fmt<KB, VB, 4>;  // slot geometry
  constexpr int nbk = (1 << KB) - 1, nbv = (1 << VB) - 1;
  float(*s_t)[256] = reinterpret_cast<float(*)[256]>(region);
  uint2* const tabk = reinterpret_cast<uint2*>(region + kAppTabOff);
  uint2* const tabv = tabk + tqq::qtab_entries(KB);
  int* const s_sh = reinterpret_cast<int*>(region + kAppShOff);
  if (wave == 0) {
    if (lane < nbk) s_t[0][lane] = tk;
    if (lane < nbv) s_t[1][lane] = tv;
    // smallest gap between consecutive boundaries, which sit one per lane
    const float tk1 = __shfl_down(tk, 1), tv1 = __shfl_down(tv, 1);
    float gk = lane + 1 < nbk ? tk1 - tk : 2.0f;
    float gv = lane + 1 < nbv ? tv1 - tv : 2.0f;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      gk = fminf(gk, __shfl_xor(gk, m));
      gv = fminf(gv, __shfl_xor(gv, m));
    }
    if (lane == 0) {
      s_sh[0] = tqq::qtab_shift(gk, KB);
      s_sh[1] = tqq::qtab_shift(gv, VB);
    }
  }
  lds_barrier();
  const int shk = __builtin_amdgcn_readfirstlane(s_sh[0]), shv = __builtin_amdgcn_readfirstlane(s_sh[1]);
  if (tid < kWG) tqq::build_qtabs<KB, VB>(s_t, shk, shv, tabk, tabv, tid);
  lds_barrier();
  if (wave < kW) {
    uint4 A[kD / 32][2];
    tqq::hadamard_operands<kD / 32>(a.signs, lane, A);
    float zero;  // an addend of 0 the compiler cannot fold, as in tq_quantize_kernel
    asm("v_mov_b32 %0, 0" : "=v"(zero));
    const int c = lane & 15, g = lane >> 4;
    const int n_rows = kH * n_list;  // (token, kv head) rows, 16 a tile
    for (int T = wave; 16 * T < n_rows; T += kW) {
      const int row = 16 * T + c;
      const bool live = row < n_rows;
      const int tok = (live ? row : n_rows - 1) / kH, h = row % kH;
      const int b = s_list[tok];
      const uint16_t* sk = a.k_new + ((int64_t)b * kH + h) * kD + 8 * g;
      const uint16_t* sv = a.v_new + ((int64_t)b * kH + h) * kD + 8 * g;
      uint4 xk[kD / 32], xv[kD / 32];
#pragma unroll
      for (int bb = 0; bb < kD / 32; ++bb) {
        xk[bb] = *reinterpret_cast<const uint4*>(sk + 32 * bb);
        xv[bb] = *reinterpret_cast<const uint4*>(sv + 32 * bb);
      }
      const int pos = a.seq_lens[b] - 1;
      const int blk = a.bs_shift >= 0 ? (pos >> a.bs_shift) : (pos / a.bs);
      const int64_t prow = (int64_t)a.bt[(int64_t)b * a.max_blocks + blk] * a.bs + (pos - blk * a.bs);
      uint8_t* const dst = live ? a.pages_w + (prow * kH + h) * F::kSB : tq_block_append_discard;
      if (shk != tqq::kQNoTable && shv != tqq::kQNoTable) {
        tqq::quantize_region<kD, KB, true, false, false>(xk, A, zero, g, F::kKCode, s_t[0], tabk, shk,
                                                          nullptr, a.rsqrt_d, dst);
        tqq::quantize_region<kD, VB, true, false, false>(xv, A, zero, g, F::kVCode, s_t[1], tabv, shv,
                                                          nullptr, a.rsqrt_d, dst + F::kVOff);
      } else {  // a codebook too fine for its table: both regions by binary search
        tqq::quantize_region<kD, KB, false, false, false>(xk, A, zero, g, F::kKCode, s_t[0], tabk, shk,
                                                           nullptr, a.rsqrt_d, dst);
        tqq::quantize_region<kD, VB, false, false, false>(xv, A, zero, g, F::kVCode, s_t[1], tabv, shv,
                                                           nullptr, a.rsqrt_d, dst + F::kVOff);
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the slots are written before any run is loaded
  }
  lds_barrier();
}

// The producer waves' part of append_tokens: its three barriers (they do none of its work).
__device__ __forceinline__ void append_barriers() {
  lds_barrier();
  lds_barrier();
  lds_barrier();
}

template <int KB, int VB, int GM>
__global__ __launch_bounds__(kThreads) void tq_decode_block_kernel(TqBlockArgs a) {
  using F = Fmt<KB, VB, GM>;
  static_assert(kAppListOff + 4 * kAppendMax <= F::kRunBytes, "fused append scratch in one run buffer");
  constexpr int kSB = F::kSB, kVOff = F::kVOff, kRowBytes = F::kRowBytes, kRunBytes = F::kRunBytes;
  constexpr int kBuf0 = F::kBuf0, QC = F::kGroupChunks, NZ = F::kNZ;
  // One LDS array placed by hand: the tables at byte 0, run buffer k at kBuf0 + k run bytes, then
  // the query region (unless the last buffer holds the queries) and the plan words.  Only the
  // producer waves have loads in flight, and they read no LDS, so the compute waves' reads need no
  // alias information to stay clear of pending loads.
  __shared__ __align__(16) uint8_t s_lds[F::kLdsBytes];
  uint2* const s_tab = reinterpret_cast<uint2*>(s_lds);
  uint8_t* const s_r0 = s_lds + kBuf0;
  uint8_t* const s_r1 = s_r0 + kRunBytes;
  uint8_t* const s_r2 = s_r1 + kRunBytes;
  uint8_t* const s_r3 = s_r2 + kRunBytes;
  uint8_t* const s_r4 = s_r3 + kRunBytes;
  int* const s_plan = reinterpret_cast<int*>(s_lds + F::kPlanOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7: kv head; 8..11: run loads
  const int t16 = lane & 15, q4 = lane >> 4;
  const int G = a.G;

  // this thread's sequence's run count for the work plan, loaded first so that it overlaps the
  // table fill
  TqSeq own{};
  if (tid < a.num_seqs) own = seq_of<false>(a, tid);

  // Centroid operand tables: entry e (a code group: coordinates 2j, 2j + 1 in its low and high
  // half) holds the fp16 high parts of both centroids, then their low parts, scaled by 2^8; copy
  // k of entry e at byte 256 e + 8 k.  The V table (if any) follows the K table.
  for (int i = tid; i < (F::kKEnt + F::kVEnt) * kCP; i += kThreads) {
    const int e = i / kCP;
    float c0, c1;
    if (e < F::kKEnt) {
      c0 = a.kc[e & ((1 << KB) - 1)];
      c1 = a.kc[e >> KB];
    } else {
      const int ev = e - F::kKEnt;
      c0 = a.vc[ev & ((1 << VB) - 1)];
      c1 = a.vc[ev >> VB];
    }
    uint32_t h0, l0, h1, l1;
    split_half(ldexpf(c0, kLutShift), h0, l0);
    split_half(ldexpf(c1, kLutShift), h1, l1);
    s_tab[i] = make_uint2(h0 | (h1 << 16), l0 | (l1 << 16));
  }
  // The run buffers are written by the loads (which the compiler does not see as stores): one
  // ordinary store keeps it from treating the array as never written there.
  if (tid == 0) s_r0[0] = 0;
  // fused append: the codebook boundaries, boundary j in lane j of wave 0 (they load with the
  // sequence lengths)
  float tk = 0.0f, tv = 0.0f;
  if (a.k_new != nullptr && wave == 0) {
    tk = a.kt[min(lane, (1 << KB) - 2)];
    tv = a.vt[min(lane, (1 << VB) - 2)];
  }
  int* const s_list = reinterpret_cast<int*>(s_r4 + kAppListOff);

  const TqPlan plan = make_plan(a, s_plan, s_list, tid, wave, lane, own);  // its barriers also cover the tables
  // fused append: the sequences whose new token this workgroup writes (the same count in every
  // wave); the compute waves quantize them before their first unit, the producers pass the same
  // barriers in theirs
  const int n_list = a.k_new != nullptr
                         ? __builtin_amdgcn_readfirstlane(min(s_plan[3 * kWaves + 7], kAppendMax)) : 0;
  bool first_unit = true;

  if (wave >= kW) {
    // ======== producer waves: every page load of the workgroup ========
    // Run r goes to buffer r mod 5 in kLoads loads of 1 KB (LDS chunks 64 k + lane); producer p
    // issues loads k = p, p + 4, ... of every run.  One wave issues such loads at about a fifth
    // of the rate the memory system serves a compute unit, so a run's loads are spread over four
    // waves.  While the compute waves read run s + 1, runs s + 2 .. s + 5 are in flight.  The
    // compute waves never issue a vector memory instruction in the loop, so a busy load path
    // stalls these waves only.
    const int pw = wave - kW;                        // producer 0..3
    const bool more = pw < F::kLoads % kNP;          // this producer issues kLoadsHi loads a run
    int src_off[F::kLoadsHi];
#pragma unroll
    for (int i = 0; i < F::kLoadsHi; ++i)
      src_off[i] = 16 * run_chunk_at<QC>(64 * min(pw + 4 * i, F::kLoads - 1) + lane);
    // wait for this wave's loads of the oldest run in flight, `later` runs being issued after it
    auto wait_later = [&](int later) {
      if (later >= 3) {
        if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * F::kLoadsHi));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * F::kLoadsLo));
      } else if (later == 2) {
        if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * F::kLoadsHi));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * F::kLoadsLo));
      } else if (later == 1) {
        if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm(F::kLoadsHi));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(F::kLoadsLo));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
    };
    for_each_unit(a, plan, [&](const TqSeq& sq, int b, int run_first, int n_run, int) {
      lds_barrier();  // every wave is done with the previous unit's buffers
      // page rows of runs run_first + lane + 64 i (clamped to the last run)
      int rows[kMaxRuns / 64];
#pragma unroll
      for (int i = 0; i < kMaxRuns / 64; ++i) rows[i] = run_row(a, b, run_first + min(lane + 64 * i, n_run - 1));
      auto issue = [&](int r, lds_u8* buf) {
        int row = __builtin_amdgcn_readlane(rows[0], r & 63);
#pragma unroll
        for (int i = 1; i < kMaxRuns / 64; ++i)
          if ((r >> 6) == i) row = __builtin_amdgcn_readlane(rows[i], r & 63);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.pages + (int64_t)row * kRowBytes, kRunBytes);
#pragma unroll
        for (int i = 0; i < F::kLoadsHi; ++i)
          if (i < F::kLoadsLo || more) lds_dma16(rs, buf + 1024 * (pw + 4 * i), src_off[i]);
      };
      // fused append (first unit): runs 0..3 go out while the compute waves quantize the new
      // tokens, unless one of them holds a new token (a unit of at most four runs ending its
      // sequence), which must wait for the slot's store.  The compute waves pass their three
      // append barriers, then this unit's start barrier: counted together with this one, the
      // stores complete at the third, before the fourth that precedes an early issue; a later
      // run holding a token is issued after the first step's barrier, the fifth.
      const bool append = first_unit && n_list > 0;
      const bool token_early = n_run <= 4 && run_first + n_run == sq.run0 + sq.n_run;
      first_unit = false;
      if (append && token_early) append_barriers();
      // runs 0..3 (the last buffer may hold the compute waves' queries until the first barrier)
      issue(0, lds_ptr(s_r0));
      if (n_run > 1) issue(1, lds_ptr(s_r1));
      if (n_run > 2) issue(2, lds_ptr(s_r2));
      if (n_run > 3) issue(3, lds_ptr(s_r3));
      if (append && !token_early) append_barriers();
      wait_later(min(n_run - 1, 3));  // run 0 is in
      lds_barrier();
      if (n_run > 4) issue(4, lds_ptr(s_r4));
      // step s: every producer waits for its loads of run s + 1, barrier (every wave is done with
      // run s), then they fetch run s + 5 into run s's buffer
      auto step = [&](int s, lds_u8* fill) {
        if (s + 1 < n_run) wait_later(min(n_run - 1, s + 4) - (s + 1));
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
    });
    return;
  }

  // ======== compute waves: wave h computes kv head h ========
  // fused append first: its three barriers precede the first unit's start barrier here, and meet
  // the producers' first unit start, then their two or three append barriers (barriers are counted,
  // not named: either way the slots are stored before the producers load a run that holds one)
  if (n_list > 0) append_tokens<KB, VB>(a, s_r4, s_list, n_list, tid, wave, lane, tk, tv);
  const int h = wave;
  const uint8_t* const tab = reinterpret_cast<const uint8_t*>(s_tab);
  const uint32_t kcopy = 8u * (uint32_t)(lane & 31);

  // ---- per-lane LDS offsets within a run buffer (the same for every run) ----
  // Each offset is held as an LDS address less kBuf0 (opaque to the compiler), so a read adds the
  // buffer's base minus kBuf0 as the DS instruction's immediate offset: no address arithmetic per
  // read for the four buffers whose base is within 64 KB of the first.
  auto lane_addr = [](int off) {
    int x = off + kBuf0;
    asm volatile("" : "+v"(x));
    return x;
  };
  // K codes of position t16, the lane's coordinates 32 q4 .. 32 q4 + 31.  4-bit codes: bytes
  // 16 q4 .. 16 q4 + 15 as two 8-byte reads, lanes with odd q4 reading the upper half first (the
  // two halves of a 32-lane pass then use distinct banks); word order w[0..1] = first read,
  // w[2..3] = second.  3-bit codes: bytes 12 q4 .. 12 q4 + 11 as three dword reads.
  const int sw = KB == 4 ? (q4 & 1) : 0;
  const int kbase = kRowBytes * t16 + kSB * h + (kD * KB / 32) * q4;
  int off_k[3];
  if constexpr (KB == 4) {
    off_k[0] = lane_addr(run_lds_offset<QC>(kbase + 8 * sw));
    off_k[1] = lane_addr(run_lds_offset<QC>(kbase + 8 * (1 - sw)));
    off_k[2] = 0;
  } else {
#pragma unroll
    for (int i = 0; i < 3; ++i) off_k[i] = lane_addr(run_lds_offset<QC>(kbase + 4 * i));
  }
  const int off_kn = lane_addr(run_lds_offset<QC>(kRowBytes * t16 + kSB * h + F::kKCode));
  const int off_vn = lane_addr(run_lds_offset<QC>(kRowBytes * t16 + kSB * h + kVOff + F::kVCode));
  // V codes of positions q4 + 4 m, m = 0..3: coordinates 8 t16 .. 8 t16 + 7 (a dword of 4-bit
  // codes, 16 bits of 2-bit codes)
  int off_v[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    off_v[m] = lane_addr(run_lds_offset<QC>(kRowBytes * (q4 + 4 * m) + kSB * h + kVOff + VB * t16));
  // read of buffer `buf` at lane address x
  auto at = [&](const uint8_t* buf, int x) { return buf - kBuf0 + x; };
  // PV weight gather: row t16 of row set z is (query head NZ (t16 >> 2) + z, coordinate (t16 >> 1)
  // & 1 of the code group, weight part t16 & 1); it takes the weights of positions q4 + 4 m from
  // softmax lane 16 (t16 >> 2) + position.
  const int bp_base = 4 * (16 * (t16 >> 2) + q4);
  const uint32_t bp_sel = ((t16 >> 1) & 1) ? ((t16 & 1) ? 0x03020c0cu : 0x01000c0cu)
                                           : ((t16 & 1) ? 0x0c0c0302u : 0x0c0c0100u);
  uint8_t* const qreg = F::kQInRing ? s_r4 + h * (kRunBytes / kW) : s_lds + F::kQBase + h * F::kQBytes;

  // ---- key half of one run: table entries of this lane's 16 code groups, and the norms ----
  auto key_codes = [&](const uint8_t* buf, uint32_t (&w)[4], float& kn, float& vn) {
    if constexpr (KB == 4) {
      const u32x2 r0 = *reinterpret_cast<const u32x2*>(at(buf, off_k[0]));
      const u32x2 r1 = *reinterpret_cast<const u32x2*>(at(buf, off_k[1]));
      w[0] = r0.x;
      w[1] = r0.y;
      w[2] = r1.x;
      w[3] = r1.y;
    } else {
#pragma unroll
      for (int i = 0; i < 3; ++i) w[i] = *reinterpret_cast<const uint32_t*>(at(buf, off_k[i]));
      w[3] = 0;
    }
    kn = *reinterpret_cast<const float*>(at(buf, off_kn));
    vn = *reinterpret_cast<const float*>(at(buf, off_vn));
  };
  auto key_lookup = [&](const uint32_t (&w)[4], uint2 (&ke)[16], int e0 = 0, int e1 = 16) {
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      uint32_t off;
      if constexpr (KB == 4) {  // byte e of the word order
        off = __builtin_amdgcn_perm(w[e >> 2], kcopy, 0x0c0c0000u | ((4u + (e & 3)) << 8));
      } else {  // bits 6 e .. 6 e + 5 of the lane's 96 code bits, moved to bits 8 .. 13
        const int P = 6 * e;
        uint32_t x;
        if (P < 8) {
          x = w[0] << (8 - P);
        } else {
          const int s = P - 8, j = s >> 5, sh = s & 31;
          x = j + 1 < 3 ? __builtin_amdgcn_alignbit(w[j + 1], w[j], sh) : (w[j] >> sh);
        }
        off = (x & 0x3f00u) | kcopy;
      }
      ke[e] = *reinterpret_cast<const uint2*>(tab + off);
    }
  };

  // value entries of one run: positions (q4, q4 + 4) then (q4 + 8, q4 + 12), code group mi of the
  // lane's 8 coordinates
  auto value_codes = [&](const uint8_t* buf, uint32_t (&cw)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if constexpr (VB == 4) cw[m] = *reinterpret_cast<const uint32_t*>(at(buf, off_v[m]));
      else cw[m] = *reinterpret_cast<const uint16_t*>(at(buf, off_v[m]));
    }
  };
  auto value_entry = [&](uint32_t x, int mi) {
    uint32_t off;
    if constexpr (VB == 4) {
      off = __builtin_amdgcn_perm(x, kcopy, 0x0c0c0000u | ((4u + mi) << 8));
    } else {  // nibble mi moved to bits 8 .. 11
      const uint32_t y = mi == 0 ? x << 8 : mi == 1 ? x << 4 : mi == 2 ? x : x >> 4;
      off = (y & 0xf00u) | kcopy;
    }
    return *reinterpret_cast<const uint2*>(tab + F::kVTab + off);
  };
  auto value_lookup = [&](const uint32_t (&cw)[4], uint2 (&ve)[16]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        ve[8 * hf + 2 * mi] = value_entry(cw[2 * hf], mi);
        ve[8 * hf + 2 * mi + 1] = value_entry(cw[2 * hf + 1], mi);
      }
    }
  };

  for_each_unit(a, plan, [&](const TqSeq& sq, int b, int run_first, int n_run, int part) {
    lds_barrier();  // every wave is done with the previous unit's buffers

    // Unit state: QK operands of the rotated queries, the softmax references and sums of the
    // lane's NZ query heads, and the PV accumulators.
    uint4 aq[8];
    float f_z[NZ], m_s[NZ], m_w[NZ], l_s[NZ], t_s[NZ], t_w[NZ], m_b[NZ];
    float4_t acc[NZ][4];
    {
      // This wave's fp16 queries (rows of 256 bytes, four per pass) into its query region, whose
      // ring buffer (if any) takes a run only after the first step's barrier.
      {
        const int64_t r0q = q_row(a, b, h, 0);
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(a.q + r0q * kD, INT_MAX);
#pragma unroll
        for (int zz = 0; zz < NZ; ++zz) {
          const int g = 4 * zz + q4 < G ? 4 * zz + q4 : 0;  // query heads past G read a live row, unused
          const int dq = (int)(q_row(a, b, h, g) - r0q) * (2 * kD) + 16 * t16;  // bytes from head row 0
          lds_dma16(rq, lds_ptr(qreg) + 1024 * zz, dq);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      // rotated queries H (s * q): pass zz, lane (g = 4 zz + q4, j = t16) holds coordinates 8 j ..
      // 8 j + 7; rotated rows as fp32 [GM][128] over the raw rows (LDS keeps this wave's order)
      float qmax_l[NZ];
      {
        float x[NZ][8];
#pragma unroll
        for (int zz = 0; zz < NZ; ++zz) {
          const uint4 raw = *reinterpret_cast<const uint4*>(qreg + 1024 * zz + 16 * lane);
          const uint32_t qw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[zz][2 * i] = half_bits_to_float(qw[i] & 0xffffu);
            x[zz][2 * i + 1] = half_bits_to_float(qw[i] >> 16);
          }
        }
        const int j = t16;
        const uint32_t swd = j < 4 ? a.signs.w[0] : j < 8 ? a.signs.w[1] : j < 12 ? a.signs.w[2] : a.signs.w[3];
        const uint32_t sb = (swd >> (8 * (j & 3))) & 0xffu;
#pragma unroll
        for (int zz = 0; zz < NZ; ++zz) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if ((sb >> e) & 1u) x[zz][e] = -x[zz][e];
          wht_row8_dpp<16>(x[zz], j);
          float mx = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[zz][e]));
          qmax_l[zz] = max16(mx) * a.qscale;
        }
#pragma unroll
        for (int zz = 0; zz < NZ; ++zz) {
          float4* d = reinterpret_cast<float4*>(qreg + 512 * (4 * zz + q4) + 32 * j);
          d[0] = make_float4(x[zz][0], x[zz][1], x[zz][2], x[zz][3]);
          d[1] = make_float4(x[zz][4], x[zz][5], x[zz][6], x[zz][7]);
        }
      }
      // scale exponent of head g: its largest |q| * qscale lands near 2^13.  (g may vary by lane:
      // each head's maximum is read from its lane as a scalar, not kept in an array the compiler
      // could turn into an indexed scratch load.)
      auto head_exp = [&](int g) {
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < GM; ++k) {
          const float qk = lane_value(qmax_l[k >> 2], 16 * (k & 3));
          v = g == k ? qk : v;
        }
        return v > 0.0f ? 13 - ilogbf(v) : 0;
      };

      // QK A operand, step mi: row t16 = (query head, fp16 part t16 & 1) -- the head t16 >> 2,
      // rows with (t16 >> 1) & 1 zero, when GM is 4, else t16 >> 1; K holds the coordinates of
      // code groups 2 mi, 2 mi + 1 of this lane's word order, [x_a, x_b, x_a, x_b, x_c, x_d, x_c,
      // x_d] against the centroid parts [hi, hi, lo, lo, hi, hi, lo, lo].
      {
        const int hd = GM == 4 ? t16 >> 2 : t16 >> 1;
        const bool live = (GM == 8 || ((t16 >> 1) & 1) == 0) && hd < G;
        const bool lo_part = t16 & 1;
        const float f = live ? ldexpf(a.qscale, head_exp(hd)) : 0.0f;
        // this lane's 32 coordinates 32 q4 .. 32 q4 + 31 in word order (upper 16 first if sw)
        const uint8_t* src = qreg + 512 * (live ? hd : 0);
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
          uint32_t pp[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t hi, lo;
            split_half(live ? x[4 * mi + i] * f : 0.0f, hi, lo);
            pp[i] = lo_part ? lo : hi;
          }
          const uint32_t ab = pp[0] | (pp[1] << 16), cd = pp[2] | (pp[3] << 16);
          aq[mi] = make_uint4(ab, ab, cd, cd);
        }
      }
      // softmax lane: position t16, query heads NZ q4 + z
#pragma unroll
      for (int z = 0; z < NZ; ++z) {
        const int g = NZ * q4 + z;
        f_z[z] = g < G ? ldexpf(1.0f, -(head_exp(g) + kLutShift)) : 0.0f;
        m_s[z] = kSent;
        m_w[z] = kSent;
        l_s[z] = 0.0f;
        t_s[z] = kSent + kThr;  // thresholds and weight base of the references
        t_w[z] = kSent + kThr;
        m_b[z] = kSent - (float)kWShift;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[z][c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }

    // position masks of the softmax lane (position t16, query heads NZ q4 + z): p >= ns, and p
    // below the packed end and the head's causal limit
    // (as one unsigned compare: p - ns < span, span = 0 for dead heads)
    const int lo_l = sq.ns - t16;
    uint32_t span[NZ];
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
      const int g = NZ * q4 + z;
      const int lim = min(sq.end, sq.seq_len - a.nq + a.q0 + g / a.g_real + 1);
      span[z] = g < G ? (uint32_t)max(lim - sq.ns, 0) : 0u;
    }

    // QK: this lane's scores (position t16, heads NZ q4 + z) before the norm and scales
    auto key_mfma = [&](const uint2 (&ke)[16], float (&sc)[NZ]) {
      float4_t sa = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        sa = mfma16(aq[mi], make_uint4(ke[2 * mi].x, ke[2 * mi].y, ke[2 * mi + 1].x, ke[2 * mi + 1].y), sa);
#pragma unroll
      for (int z = 0; z < NZ; ++z) sc[z] = sa[2 * z] + sa[2 * z + 1];
    };

    // Pipeline state carried from step s - 1: run s's raw scores and norms (position t16) and its
    // value entries.  Step s issues run s + 1's key lookups, then does run s's softmax and PV,
    // then issues run s + 1's value lookups (after PV has consumed run s's) and does run s + 1's
    // QK.  Table lookups stay in flight across the step barrier; every read of a run buffer is
    // consumed within its step, before the barrier that can release the buffer.
    float sc[NZ], knf[NZ], lv = 0.0f;  // run s: raw scores, n_K * f_z, log2 n_V (position t16)
    uint2 ve[16];
    auto body = [&](int s, const uint8_t* nxt) {
      uint32_t kw[4], cw[4];
      float kn1, vn1;
      key_codes(nxt, kw, kn1, vn1);
      value_codes(nxt, cw);
      __builtin_amdgcn_sched_barrier(0);  // the code reads go out first
      uint2 ke[16];
      // With eight query heads the second half of the key lookups waits until PV has used this
      // run's value entries (registers)
      key_lookup(kw, ke, 0, NZ == 1 ? 16 : 8);

      // softmax of run s, lane (position t16, heads NZ q4 + z); masked rows never touch their
      // garbage norms.  The references m_s (scores) and m_w (scores + log2 n_V) move only when
      // some score passes them by more than kThr: terms stay below 2^kThr, weights below
      // 2^(kWShift + kThr).
      const int pb = (run_first + s) * 16;
      float s0[NZ], sw0[NZ];
      bool over = false;
#pragma unroll
      for (int z = 0; z < NZ; ++z) {
        const bool valid = (uint32_t)(pb - lo_l) < span[z];
        s0[z] = valid ? sc[z] * knf[z] : -INFINITY;
        sw0[z] = valid ? s0[z] + lv : -INFINITY;  // + log2(n_V)
        // (eight heads: the thresholds are recomputed, which saves their registers)
        if constexpr (NZ == 1) over = over || s0[z] > t_s[z] || sw0[z] > t_w[z];
        else over = over || s0[z] > m_s[z] + kThr || sw0[z] > m_w[z] + kThr;
      }
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
        for (int z = 0; z < NZ; ++z) {
          const float ns2 = fmaxf(m_s[z], max16(s0[z])), nw2 = fmaxf(m_w[z], max16(sw0[z]));
          l_s[z] *= __builtin_amdgcn_exp2f(m_s[z] - ns2);
          const float r = __builtin_amdgcn_exp2f(m_w[z] - nw2);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[z][c] *= r;
          m_s[z] = ns2;
          m_w[z] = nw2;
          t_s[z] = ns2 + kThr;
          t_w[z] = nw2 + kThr;
          m_b[z] = nw2 - (float)kWShift;
        }
      }
#pragma unroll
      for (int z = 0; z < NZ; ++z) {
        l_s[z] += __builtin_amdgcn_exp2f(s0[z] - m_s[z]);
        const float wt = __builtin_amdgcn_exp2f(sw0[z] - (NZ == 1 ? m_b[z] : m_w[z] - (float)kWShift));
        const auto h2 = __builtin_amdgcn_cvt_pkrtz(wt, 0.0f);
        const auto p2 = __builtin_amdgcn_cvt_pkrtz(wt, wt - (float)h2[0]);
        const uint32_t wpk = __builtin_bit_cast(uint32_t, p2);  // both fp16 parts of the weight

        // PV A operands: positions q4 + 4 m of head NZ (t16 >> 2) + z, one weight part, at the
        // row's coordinate of the code group
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
            acc[z][mi] = mfma16(aw, make_uint4(e0.x, e0.y, e1.x, e1.y), acc[z][mi]);
          }
        }
      }
      if constexpr (NZ == 1) {
        value_lookup(cw, ve);  // run s + 1
        key_mfma(ke, sc);
      } else {  // the value lookups follow QK and stay in flight across the barrier
        key_lookup(kw, ke, 8, 16);
        key_mfma(ke, sc);
        value_lookup(cw, ve);
      }
      // the norms of run s + 1 are used here, so no read of its buffer outlives the step
#pragma unroll
      for (int z = 0; z < NZ; ++z) knf[z] = kn1 * f_z[z];
      lv = __builtin_amdgcn_logf(vn1);
    };

    lds_barrier();  // run 0 is in
    {
      uint32_t kw[4], cw[4];
      uint2 ke[16];
      float kn0, vn0;
      key_codes(s_r0, kw, kn0, vn0);
      value_codes(s_r0, cw);
      key_lookup(kw, ke);
      value_lookup(cw, ve);
      key_mfma(ke, sc);
#pragma unroll
      for (int z = 0; z < NZ; ++z) knf[z] = kn0 * f_z[z];
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

    {
      // ---- this wave's partials for heads NZ q4 + z: coordinates 8 t16 + 2 mi + (0, 1) ----
#pragma unroll
      for (int z = 0; z < NZ; ++z) {
        const int g = NZ * q4 + z;
        const float ls = sum16(l_s[z]);
        if (g < G) {
          const float c0 = __builtin_amdgcn_exp2f(m_w[z] - m_s[z]) * ldexpf(1.0f, -(kWShift + kLutShift));
          float* pt = a.partials + ((((int64_t)b * kH + h) * a.part_stride + part) * G + g) * (kD + 2);
          float2* o = reinterpret_cast<float2*>(pt + 2 + 8 * t16);
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
            o[mi] = make_float2((acc[z][mi][0] + acc[z][mi][1]) * c0, (acc[z][mi][2] + acc[z][mi][3]) * c0);
          if (t16 == 0) *reinterpret_cast<float2*>(pt) = make_float2(m_s[z], ls);
        }
      }
    }
  });
}

template <int KB, int VB, int GM>
void launch_block(const TqBlockArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((tq_decode_block_kernel<KB, VB, GM>), dim3(kGrid), dim3(kThreads), 0, st, a);
}

}  // namespace

// Whether the block-streaming kernel serves a format: D = 128, eight kv heads, unpadded plain
// slots (norm correction changes the stored norm only), page blocks of whole 16-position runs;
// K4/V4 with one codebook array for keys and values and at most four query heads per kv head, or
// K3/V2 with at most eight.
bool tq_decode_block_format(const TqLayer& L) {
  if (!(L.D == 128 && L.Hkv == kH && L.stride == L.slot_bytes && !L.mean && !L.qjl && L.bs % 16 == 0))
    return false;
  if (L.kb == 4 && L.vb == 4) return L.G <= 4 && L.kc == L.vc;
  if (L.kb == 3 && L.vb == 2) return L.G <= 8;
  return false;
}

// Work geometry of the block kernel.  max_runs bounds a sequence's runs; max_pieces bounds the
// workgroups one sequence spans: enough that the workgroups can share a few long sequences evenly,
// few enough that a large batch keeps a small workspace.  max_split bounds its partials (per
// sequence and kv head).
TqSplit tq_decode_block_split(int num_seqs, int max_seq_len) {
  const long runs = max_seq_len > 0 ? ((long)max_seq_len + 15) / 16 : 1;
  const long ns = num_seqs > 0 ? num_seqs : 1;
  long pieces = (2L * kGrid + ns - 1) / ns + 2;
  if (pieces > runs + 2) pieces = runs + 2;
  if (pieces < 3) pieces = 3;
  TqSplit sp;
  sp.chunk = 16;
  sp.max_pieces = (int)pieces;
  // partials: a unit of at most kMaxRuns runs each, pieces - 1 pieces at most
  sp.max_split = (int)(pieces + (runs + kMaxRuns - 1) / kMaxRuns);
  sp.max_runs = (int)runs;
  return sp;
}

int tq_launch_decode_block(const TqLayer& L, const void* q, const void* pages, const int32_t* block_tables,
                           int max_blocks, const int32_t* seq_lens, int num_seqs, const TqSplit& sp,
                           int n_sink, const int32_t* win_lens, int win_cap, float qscale, float* partials,
                           int32_t* nsplit, int part_stride, int nq, int q0, int g_real, void* stream,
                           const TqAppend* app) {
  if (sp.max_pieces < 3 || sp.max_runs < 1 || sp.max_split < sp.max_pieces || part_stride < sp.max_split)
    return (int)hipErrorInvalidValue;
  TqBlockArgs a;
  a.q = (const uint16_t*)q;
  a.pages = (const uint8_t*)pages;
  a.bt = block_tables;
  a.seq_lens = seq_lens;
  a.win_lens = win_cap > 0 ? win_lens : nullptr;
  a.partials = partials;
  a.nsplit = nsplit;
  a.kc = L.kc;
  a.vc = L.vc;
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
  a.num_seqs = num_seqs;
  a.part_stride = part_stride;
  a.max_pieces = sp.max_pieces;
  a.max_parts = sp.max_split;
  a.max_runs = sp.max_runs;
  a.nq = nq;
  a.q0 = q0;
  a.g_real = g_real;
  a.k_new = app != nullptr ? (const uint16_t*)app->k : nullptr;
  a.v_new = app != nullptr ? (const uint16_t*)app->v : nullptr;
  a.pages_w = app != nullptr ? (uint8_t*)app->pages : nullptr;
  a.kt = L.kt;
  a.vt = L.vt;
  a.rsqrt_d = (float)(1.0 / __builtin_sqrt((double)kD));  // as tq_quantize_kernel takes it
  const hipStream_t st = (hipStream_t)stream;
  if (L.kb == 4) launch_block<4, 4, 4>(a, st);
  else if (L.G <= 4) launch_block<3, 2, 4>(a, st);
  else launch_block<3, 2, 8>(a, st);
  return (int)hipGetLastError();
}
