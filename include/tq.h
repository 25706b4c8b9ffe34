/*
 * tq.h — C ABI of the TurboQuant packed-KV library for AMD Instinct MI355X (gfx950).
 *
 * Two halves of one hot path, as the pages describe it:
 *   1. quantize-on-append: randomized Hadamard rotation (sign flip + Walsh-Hadamard transform),
 *      fp32 L2-norm split, nearest Lloyd-Max centroid per rotated coordinate, and bit packing of
 *      the indices plus the norm into TQ page slots
 *      (turboquant-serve 0.1.2, "Architecture"; turboquant-pro 1.4.2, "How It Works";
 *       tq-kv, "How It Works" step [3]; TorbuQuant docs, "TQ4 page tensor" figure);
 *   2. fused paged decode attention that reads the packed pages directly: scores on the codes
 *      with a rotated query, online softmax, values accumulated in the rotated domain and rotated
 *      back once per output (tq-kv, "Quick Start" pre_rotate_query_with_signs /
 *      fused_attention_scores and "Custom CUDA Kernel Stack" split-KV flash decode;
 *      turboquant-pro 1.4.2, "Fused CUDA decode").
 *
 * Page layout (TorbuQuant docs, "TQ4 page tensor" figure): a uint8 tensor
 *   pages[num_blocks][block_size][num_kv_heads][slot_stride]
 * The slot of token position p of a sequence is slot = block_table[p / block_size] * block_size
 * + p % block_size, and kv head h of that slot starts at byte (slot * num_kv_heads + h) *
 * slot_stride.  Each slot holds a K region then a V region; a region is ceil(D * bits / 8) bytes
 * of indices (LSB-first bitstream: index i occupies bits [i*bits, (i+1)*bits), byte k holds bits
 * 8k..8k+7) followed by the row's fp32 L2 norm, little-endian.  Bytes from slot_bytes up to
 * slot_stride are written as zero.
 *
 * Conventions for every call below:
 *   - Pointers marked "device" are device memory of the current HIP device; the caller owns
 *     them and keeps them alive until the stream has finished the work.  The library never
 *     allocates or frees device memory and keeps no pointer after a call returns.  (Its one
 *     device array, the static workspace of tq_paged_decode_attention_noalloc, is part of the
 *     loaded code object.)
 *   - Calls that take a stream only enqueue work on it and return without waiting.
 *   - Every argument is validated on the host before anything is enqueued.  A call returns
 *     TQ_OK (0) or a negative tq_status; on error nothing was enqueued.  No exception crosses
 *     the ABI.  Device-side contract violations (a block id >= num_blocks, seq_len >
 *     max_seq_len, a slot >= num_blocks * block_size, duplicate slots in one append,
 *     non-finite inputs) are undefined behaviour.
 *   - fp16 means IEEE binary16 stored as uint16; fp32 means IEEE binary32.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef TQ_STREAM_T_DEFINED
#define TQ_STREAM_T_DEFINED
typedef struct ihipStream_t* tq_stream_t; /* a hipStream_t; NULL = the default stream */
#endif

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,    /* a null pointer, a negative size, H_q % H_kv != 0, ...       */
  TQ_ERR_UNSUPPORTED = -2,    /* head_dim, bit width or a size outside what the kernels       *
                               * implement (a launch grid beyond 32-bit workgroup counts)     */
  TQ_ERR_WORKSPACE = -3,      /* decode workspace smaller than tq_decode_workspace_bytes()   */
  TQ_ERR_HIP = -4,            /* the HIP runtime reported an error while enqueueing          */
  TQ_ERR_NO_CONVERGENCE = -5, /* the Lloyd-Max solver did not reach its tolerance            */
  TQ_ERR_NOALLOC_LIMIT = -6   /* the sizes need more workspace than the library's static     *
                               * array holds (tq_paged_decode_attention_noalloc)              */
} tq_status;

typedef enum tq_codebook_family {
  TQ_CODEBOOK_BETA = 0,     /* exact law of one coordinate of a uniform point on S^{D-1}   */
  TQ_CODEBOOK_GAUSSIAN = 1  /* its N(0, 1/D) approximation                                  */
} tq_codebook_family;

/* Format flags of tq_layer_desc.flags.
 *   TQ_FLAG_NORM_CORRECTION  (tq-kv, "How It Works": Lloyd-Max codebook + norm correction, output
 *   "corrected norm") each region stores n / ||c[idx]||_2 instead of n = ||x||_2, so the
 *   dequantized row n' R^T c[idx] keeps the input row's L2 norm.  ||c[idx]||^2 is summed in fp32
 *   by the stride-halving tree over the rotated coordinates (pairs i, i + D/2 first) of the
 *   fp32-rounded squares; the square root and the division are correctly rounded; a zero row
 *   keeps a zero norm.  Only tq_quantize_append changes: decode and dequantize read the stored
 *   norm as it is.
 *   TQ_FLAG_MEAN_REMOVAL  (tq-kv, "How It Works": per-token mean removal, and the mean in the
 *   output record) each region stores the row mean mu as a second fp32 after the norm (region
 *   bytes ceil(D*bits/8) + 8; see tq_slot_bytes_ex).  mu is the stride-halving fp32 tree sum of
 *   the row divided by D; the row is centred, d = fp32(x - mu), n is the norm of d (fp32-rounded
 *   squares, the same tree, correctly rounded sqrt) and the codes encode R d / n.  The
 *   dequantized row is fp32(x_hat + mu), so decode adds mu * sum(q) to each score and the
 *   weighted means to each output.  Combines with TQ_FLAG_NORM_CORRECTION (which then corrects
 *   the norm of d).
 *   TQ_FLAG_QJL  (tq-kv, "How It Works": step [5], SRHT QJL error correction; TorbuQuant docs,
 *   "Current Status": QJL residual; the TurboQuant and QJL papers in the TorbuQuant references)
 *   keys of 2, 3 or 4 bits also carry a 1-bit sketch of their quantization residual.  In the
 *   rotated frame the residual is r = R (x - mu 1) - n_s c[idx] (n_s the stored norm); the key
 *   region gains, after its norm (and mean), D/8 bytes holding b_i = [(S r)_i >= 0] LSB-first and
 *   then gamma = ||r||_2 as fp32, where S = H_D diag(sigma2) and sigma2 is the SplitMix64 sign
 *   vector of rht_seed XOR 0x514A4C5F534B4554.  The dequantized key gains
 *   sqrt(pi/2) / D * gamma * R^T S^T (2 b - 1), so decode adds
 *   scale * sqrt(pi/2) / D * gamma * (S R q) . (2 b - 1) to each score.  Values are unchanged.
 *   r, gamma and S r are formed in fp64 (R (x - mu 1) as an exact Walsh-Hadamard transform of the
 *   fp16 row times fp64(1/sqrt(D))): a bit whose |(S r)_i| is within about 1e-12 gamma of 0, or a
 *   gamma within that distance of an fp32 rounding midpoint, may differ from an exact
 *   computation.  Combines with the other flags.
 * Other bits must be 0. */
#define TQ_FLAG_NORM_CORRECTION 1
#define TQ_FLAG_MEAN_REMOVAL 2
#define TQ_FLAG_QJL 4

/* One layer's format.  K and V may use different bit widths (tiny-turboquant 0.12.0.3,
 * "Current status": q8k-q8v and q8k-int4v policies; TorbuQuant docs, "Current Status": K8/K4 and
 * V8/V4/V3/V2 formats); a model with boundary-layer protection simply uses a different
 * descriptor for the protected layers. */
typedef struct tq_layer_desc {
  int32_t head_dim;       /* D: 64 or 128                                                     */
  int32_t num_q_heads;    /* H_q (decode only; multiple of num_kv_heads; G = H_q/H_kv <= 8)   */
  int32_t num_kv_heads;   /* H_kv >= 1                                                         */
  int32_t block_size;     /* tokens per page block, >= 1                                       */
  int32_t k_bits;         /* 2, 3, 4 or 8                                                      */
  int32_t v_bits;         /* 2, 3, 4 or 8                                                      */
  int32_t slot_stride;    /* bytes per (token, kv head) slot; 0 means tq_slot_bytes()          */
  int32_t flags;          /* format flags (TQ_FLAG_*), 0 for the plain format                  */
  uint64_t rht_seed;      /* seed of the SplitMix64 sign vector of the rotation                */
  const float* k_centroids;   /* device, 2^k_bits ascending fp32 (tq_build_codebook output) */
  const float* k_boundaries;  /* device, 2^k_bits - 1 ascending fp32                          */
  const float* v_centroids;   /* device, 2^v_bits                                             */
  const float* v_boundaries;  /* device, 2^v_bits - 1                                         */
} tq_layer_desc;

/* Lloyd-Max codebook for one rotated coordinate (host only, pure, no device work).
 * Follows turboquant-serve 0.1.2, "Architecture" (MSE-optimal codebook for the Beta prior on
 * rotated unit vectors, fitted once and shared) and the TorbuQuant docs, "Current Status" table
 * (exact Beta-sphere and Gaussian-approximation codebooks).  Solves the midpoint and centroid
 * conditions in fp64 to a centroid residual <= 1e-13, exactly symmetric, and rounds centroids
 * and boundaries to fp32 independently.
 *   D            head dimension, 2..65536
 *   bits         1..8
 *   family       tq_codebook_family
 *   centroids    host out, 2^bits fp32 (ascending)
 *   boundaries   host out, 2^bits - 1 fp32 (ascending; the middle one is exactly 0)
 *   centroids_f64, boundaries_f64, mse   optional host outs (NULL to skip): the fp64 fixed
 *                point and the mean squared error per coordinate. */
int tq_build_codebook(int32_t D, int32_t bits, int32_t family, float* centroids, float* boundaries,
                      double* centroids_f64, double* boundaries_f64, double* mse);

/* The rotation's sign vector (host only): signs[i] = -1 when bit 63 of the i-th SplitMix64
 * draw from `seed` is set, else +1 (tq-kv, "Quick Start": generate_signs(dim, seed)).
 * out: host, D int8 values. */
int tq_rht_signs(int32_t D, uint64_t seed, int8_t* out);

/* Bytes of one slot: (ceil(D*k_bits/8) + 4) + (ceil(D*v_bits/8) + 4) (TorbuQuant docs,
 * "TQ4 page tensor" figure).  Returns a negative tq_status for unsupported arguments. */
int32_t tq_slot_bytes(int32_t D, int32_t k_bits, int32_t v_bits);

/* Bytes of one slot of a format with flags (TQ_FLAG_*): each region gains 4 bytes with
 * TQ_FLAG_MEAN_REMOVAL, the key region D/8 + 4 bytes with TQ_FLAG_QJL (D a multiple of 8).
 * Returns a negative tq_status for unsupported arguments or flags. */
int32_t tq_slot_bytes_ex(int32_t D, int32_t k_bits, int32_t v_bits, int32_t flags);

/* Quantize-on-append (turboquant-serve 0.1.2, "Architecture" update(); TorbuQuant docs,
 * "TQ4 page tensor" figure; turboquant-pro 1.4.2, "How It Works" per-vector flow).
 *   k, v          device fp16 [n_tok][num_kv_heads][D], contiguous
 *   slot_mapping  device int64 [n_tok]: destination slot of each token; a negative slot skips
 *                 the token (padding).  Slots must be distinct and < num_blocks * block_size.
 *   pages         device uint8 [num_blocks][block_size][num_kv_heads][slot_stride] (written)
 * For each (token, kv head) and for K and V: n = fp32 norm of the fp16 row (exact squares,
 * stride-halving fp32 tree, correctly rounded sqrt); u = R x / n; index = number of fp32
 * boundaries <= u (all indices 2^bits/2 when n == 0); pack; store. */
int tq_quantize_append(const tq_layer_desc* layer, const void* k, const void* v,
                       const int64_t* slot_mapping, int64_t n_tok, void* pages, int64_t num_blocks,
                       tq_stream_t stream);

/* Workspace bytes tq_paged_decode_attention needs for these sizes: the split-K partial results
 * (running max, sum and rotated accumulator per sequence, query head and split).  It needs no
 * initialisation.  Calls sharing a workspace must be ordered on one stream. */
size_t tq_decode_workspace_bytes(const tq_layer_desc* layer, int32_t num_seqs, int32_t max_seq_len);

/* Fused paged decode attention over packed pages, one query token per sequence.
 * (tq-kv, "Custom CUDA Kernel Stack": split-KV flash decode with online softmax and TQ fused
 *  attention on compressed KV; "3-Fix for GGUF Models": sink tokens kept fp16;
 *  turboquant-pro 1.4.2, "Fused CUDA decode": split-K decode on the codes.)
 *   q             device fp16 [num_seqs][num_q_heads][D]
 *   pages         device uint8 page tensor (read only)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *                 (pages and block_tables may be NULL when max_seq_len <= n_sink: every position
 *                 is then a sink token)
 *   seq_lens      device int32 [num_seqs]: cached tokens of each sequence, sinks included;
 *                 each <= max_seq_len (a host value used to size the grid)
 *   sink_k, sink_v device fp16 [num_seqs][n_sink][num_kv_heads][D], or NULL when n_sink == 0.
 *                 Positions p < min(n_sink, seq_len) are read from these arrays; their page
 *                 slots are ignored.
 *   scale         softmax scale; <= 0 selects 1/sqrt(D)
 *   out           device fp32 [num_seqs][num_q_heads][D] (written; seq_len == 0 gives zeros)
 *   workspace     device, >= tq_decode_workspace_bytes(layer, num_seqs, max_seq_len)
 * Query head h reads kv head h / G (G = num_q_heads / num_kv_heads).  Computes, for every
 * sequence and query head, softmax(scale * q . k_p) weighted sum of v_p over p < seq_len, where
 * k_p, v_p are the sinks or the dequantized rows n R^T c[idx]; scores use n (R q) . c[idx] and
 * values are summed as n c[idx] in the rotated domain and rotated back once. */
int tq_paged_decode_attention(const tq_layer_desc* layer, const void* q, const void* pages,
                              int64_t num_blocks, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                              int32_t max_seq_len, const void* sink_k, const void* sink_v,
                              int32_t n_sink, float scale, float* out, void* workspace,
                              size_t workspace_bytes, tq_stream_t stream);

/* The same decode for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc): the split-K partials go to a static device
 * array that the library holds per GPU, TQ_NOALLOC_WORKSPACE_BYTES bytes, loaded with the library
 * and kept until the process ends.  The call allocates nothing; the caller still passes every
 * input and output.  Arguments are those of tq_paged_decode_attention without the workspace.
 * Returns TQ_ERR_NOALLOC_LIMIT when the sizes need more than the array holds (the partials of
 * num_seqs * num_kv_heads * num_q_heads/num_kv_heads * (D + 2) fp32 per split, with about three
 * splits per compute unit of the batch; e.g. 256 sequences x 8 kv heads x 8 query heads per kv
 * head at D = 128 take 17 MB), TQ_ERR_HIP when the array's address cannot be obtained.
 * Every call on one GPU shares its array: calls that may overlap on one GPU (on different
 * streams, or from several threads) race and must be ordered by the caller; calls on one stream
 * are ordered by it.  The array needs no clearing: each call writes what it reads. */
#define TQ_NOALLOC_WORKSPACE_BYTES (64u << 20)
int tq_paged_decode_attention_noalloc(const tq_layer_desc* layer, const void* q, const void* pages,
                                      int64_t num_blocks, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                      int32_t num_seqs, int32_t max_seq_len, const void* sink_k,
                                      const void* sink_v, int32_t n_sink, float scale, float* out,
                                      tq_stream_t stream);

/* One decode step's append and attention in one call: for every sequence b with seq_lens[b] >= 1,
 * the new token's K and V rows are quantized into the page slot of position seq_lens[b] - 1 (the
 * slot the block table gives that position), then decode attention runs as
 * tq_paged_decode_attention with no sink tokens.  Pages and output are identical, byte for byte,
 * to tq_quantize_append of those rows at those slots followed by tq_paged_decode_attention.
 * (turboquant-serve 0.1.2, "Architecture": each new row is rotated, normalised, encoded and packed
 *  as it is stored; tq-kv, "Custom CUDA Kernel Stack": split-KV flash decode on the compressed
 *  pages.)  The quantization is done by the decode kernel itself, by the workgroup that reads the
 *  new token's run (of that kv head, in the split-kernel formats), before it loads any run, so the
 *  step costs no separate launch.
 *   k_new, v_new  device fp16 [num_seqs][num_kv_heads][D]: the new token's rows; seq_lens counts
 *                 the new token
 *   pages         device, written (the new slots) and read
 * Other arguments as for tq_paged_decode_attention.  TQ_ERR_UNSUPPORTED unless no format flag is
 * set, the block size is a multiple of 16, num_seqs <= TQ_APPEND_MAX_SEQS, and the layer is one the
 * whole-block decode kernel serves (D = 128, eight kv heads, unpadded slots, K4/V4 with one
 * codebook for K and V and up to four query heads per kv head, or K3/V2 with up to eight) or one
 * the matrix-core split kernel serves (D = 128 with K codes of 2, 3, 4 or 8 bits and V codes of 2,
 * 4 or 8 bits; D = 64 with K and V codes of 4 or 8 bits); other callers use tq_quantize_append
 * and tq_paged_decode_attention.  The workspace is that of tq_decode_workspace_bytes. */
#define TQ_APPEND_MAX_SEQS 512
int tq_paged_decode_attention_append(const tq_layer_desc* layer, const void* q, const void* k_new,
                                     const void* v_new, void* pages, int64_t num_blocks,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                     float scale, float* out, void* workspace, size_t workspace_bytes,
                                     tq_stream_t stream);

/* The same decode with an fp16 hot window: the most recent tokens of each sequence kept
 * uncompressed and merged with the packed tokens by online softmax.
 * (turboquant-pro 1.4.2, "Streaming cache": an uncompressed hot window of recent tokens in front of
 *  the bit-packed older ones; "Fused CUDA decode": the fp16 hot window merged via online softmax;
 *  tq-kv, "3-Fix for GGUF Models": the current token kept lossless.)
 *   win_k, win_v  device fp16 [num_seqs][win_cap][num_kv_heads][D]: rows 0 .. win_lens[b] - 1 of
 *                 sequence b are its last win_lens[b] positions, in any order (attention does not
 *                 depend on the order of its tokens); their page slots are ignored
 *   win_lens      device int32 [num_seqs]: 0 <= win_lens[b] <= min(win_cap,
 *                 seq_lens[b] - min(n_sink, seq_lens[b])); values outside are clamped to it
 *   win_cap       rows per sequence in win_k / win_v, 0 .. 1024 (0: no window; then the window
 *                 pointers may be NULL)
 * Every other argument, the workspace size included, is as for tq_paged_decode_attention.  The
 * packed positions of sequence b are n_sink .. seq_lens[b] - win_lens[b] - 1. */
int tq_paged_decode_attention_window(const tq_layer_desc* layer, const void* q, const void* pages,
                                     int64_t num_blocks, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     int32_t num_seqs, int32_t max_seq_len, const void* sink_k,
                                     const void* sink_v, int32_t n_sink, const void* win_k,
                                     const void* win_v, const int32_t* win_lens, int32_t win_cap,
                                     float scale, float* out, void* workspace,
                                     size_t workspace_bytes, tq_stream_t stream);

/* Decode several query tokens per sequence at once, in causal order: the last n_queries cached
 * positions of each sequence are the new tokens (their rows already appended), e.g. a draft being
 * verified or a chunk of a prompt.
 * (tq-kv, "What's next": attention over more than the single decode token, for prefill, and the
 *  verification of EAGLE draft tokens.)
 *   q             device fp16 [num_seqs][n_queries][num_q_heads][D]
 *   n_queries     1 .. TQ_MAX_QUERIES
 *   out           device fp32 [num_seqs][n_queries][num_q_heads][D] (written)
 *   workspace     device, >= tq_decode_multi_workspace_bytes(layer, num_seqs, max_seq_len,
 *                 n_queries)
 * Query j of sequence b sits at position seq_lens[b] - n_queries + j and attends positions 0 ..
 * seq_lens[b] - n_queries + j: the single-query result over that many cached tokens (a query at a
 * negative position gives zeros).  Sinks are as for tq_paged_decode_attention; there is no hot
 * window.  The page bytes are read once for up to 8 / G queries (G query heads per kv head) and
 * once more per further group of queries.  Other arguments as for tq_paged_decode_attention. */
#define TQ_MAX_QUERIES 64
size_t tq_decode_multi_workspace_bytes(const tq_layer_desc* layer, int32_t num_seqs,
                                       int32_t max_seq_len, int32_t n_queries);
int tq_paged_decode_attention_multi(const tq_layer_desc* layer, const void* q, int32_t n_queries,
                                    const void* pages, int64_t num_blocks,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* seq_lens, int32_t num_seqs,
                                    int32_t max_seq_len, const void* sink_k, const void* sink_v,
                                    int32_t n_sink, float scale, float* out, void* workspace,
                                    size_t workspace_bytes, tq_stream_t stream);

/* Dequantize whole slots (turboquant-serve 0.1.2, "Architecture" _decode(): unpack, Lloyd-Max
 * decode, restore magnitude, rotate back).  Bit-exact definition: c_i = centroid[idx_i] (fp32);
 * z = H c computed exactly (fp64); g = fp32(n * fp32(1/sqrt(D))); x_i = s_i * fp32(fp32(z_i) * g),
 * then fp32(x_i + mu) with TQ_FLAG_MEAN_REMOVAL.  With TQ_FLAG_QJL a key also gains its sketched
 * residual: t = H diag(sigma2) H (2b - 1) exactly (fp64), and
 * x_i = s_i * fp32(fp32(fp32(z_i) * g) + fp32(fp32(t_i) * gq)), gq = fp32(sqrt(pi/2) / D * gamma *
 * fp32(1/sqrt(D))) (the product in fp64).
 *   slots         device int64 [n]: slot ids (< num_blocks * block_size)
 *   k_out, v_out  device fp32 [n][num_kv_heads][D] (written) */
int tq_dequantize_rows(const tq_layer_desc* layer, const void* pages, int64_t num_blocks,
                       const int64_t* slots, int64_t n, float* k_out, float* v_out,
                       tq_stream_t stream);

/* Static description of a status code. */
const char* tq_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
