// Internal declarations shared by the C ABI layer (tq_api.cpp), the host set-up code
// (tq_codebook.cpp) and the kernels (tq_kernels.hip).  Not part of the public ABI.
#ifndef TQ_INTERNAL_H_
#define TQ_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

// Sign bits of the rotation for head dimension D (bit i set: s_i = -1), nwords 64-bit words.
void tq_sign_words(int32_t D, uint64_t seed, uint64_t* words, int nwords);

// Largest n_sink and hot-window capacity the decode kernel accepts (their scores live in LDS).
#define TQ_MAX_SINKS 128
#define TQ_MAX_WINDOW 1024

// Fixed cost, in runs of 16 positions, that the block decode kernel's work plan charges a
// workgroup for each unit it starts (its queries, block-table rows and first runs load before it
// computes): about 11 us per unit against about 1.05 us per run of the ragged K3/V2 batch.
constexpr int kTqUnitCostRuns = 10;

// Sign bits as passed to the kernels by value (D <= 128).
struct TqSigns {
  uint32_t w[4];
};

// Validated launch parameters shared by the launchers.
struct TqLayer {
  int D, Hq, Hkv, G, bs, kb, vb;
  int stride;          // slot stride in bytes
  int slot_bytes;      // K region + V region
  int kcode_bytes;     // ceil(D * kb / 8)
  int vcode_bytes;     // ceil(D * vb / 8)
  int norm_corr;       // 1: the stored norm is n / ||c[idx]|| (norm-correction format)
  int mean;            // 1: each region ends with the row mean (mean-removal format)
  int qjl;             // 1: keys carry a 1-bit residual sketch and its norm (QJL key format)
  int kqjl;            // offset of the sketch bits in the slot (gamma follows them)
  int kreg;            // K region bytes: codes, norm (and mean), sketch; the V region starts here
  TqSigns signs;
  TqSigns signs2;      // sign vector of the residual sketch (QJL key format)
  const float *kc, *kt, *vc, *vt;
};

// Decode split geometry chosen on the host.
struct TqSplit {
  int chunk;          // page tokens per split
  int max_split;      // splits per (sequence, kv head) at max_seq_len (block kernel: pieces)
  int max_runs = 0;   // block kernel: 16-position runs of a sequence at max_seq_len
  int max_pieces = 0; // block kernel: workgroups one sequence may span, plus two
};

TqSplit tq_decode_split(const TqLayer& L, int num_seqs, int max_seq_len);
// Workspace bytes for the largest sink count and window (the public size), and for a given call.
size_t tq_decode_ws_bytes(const TqLayer& L, int num_seqs, const TqSplit& sp);
size_t tq_decode_ws_bytes_for(const TqLayer& L, int num_seqs, const TqSplit& sp, int n_sink, int win_cap);
// Device address of the library's static decode workspace on the current device (a hipError_t
// value, 0 on success).
int tq_noalloc_workspace(void** ptr);

// Fused append of tq_paged_decode_attention_append: the new token of each sequence (K and V rows
// [num_seqs][Hkv][D] fp16), quantized into the page slot of its position seq_len - 1.
struct TqAppend {
  const void* k;
  const void* v;
  void* pages;
};

// Formats whose decode call also takes the step's append (tq_paged_decode_attention_append).
bool tq_decode_append_format(const TqLayer& L);

// The whole-block streaming decode kernel (tq_decode_block.hip): the formats it serves, its split
// geometry and its launch (the split kernel only; the caller launches fp16-row chunks and merge).
bool tq_decode_block_format(const TqLayer& L);
TqSplit tq_decode_block_split(int num_seqs, int max_seq_len);
int tq_launch_decode_block(const TqLayer& L, const void* q, const void* pages, const int32_t* block_tables,
                           int max_blocks, const int32_t* seq_lens, int num_seqs, const TqSplit& sp,
                           int n_sink, const int32_t* win_lens, int win_cap, float qscale, float* partials,
                           int32_t* nsplit, int part_stride, int nq, int q0, int g_real, void* stream,
                           const TqAppend* app = nullptr);

// Launchers: return a hipError_t value (0 on success).
int tq_launch_quantize(const TqLayer& L, const void* k, const void* v, const int64_t* slot_mapping,
                       int64_t n_tok, void* pages, void* stream);
int tq_launch_decode(const TqLayer& L, const void* q, const void* pages, const int32_t* block_tables,
                     int max_blocks, const int32_t* seq_lens, int num_seqs, const TqSplit& sp,
                     const void* sink_k, const void* sink_v, int n_sink, const void* win_k,
                     const void* win_v, const int32_t* win_lens, int win_cap, float scale,
                     float* out, void* workspace, void* stream, int nq = 1, int q0 = 0,
                     int g_real = 0, const TqAppend* app = nullptr);
int tq_launch_dequant(const TqLayer& L, const void* pages, const int64_t* slots, int64_t n,
                      float* k_out, float* v_out, void* stream);

#endif  // TQ_INTERNAL_H_
