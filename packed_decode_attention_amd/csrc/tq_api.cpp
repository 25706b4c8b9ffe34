// C ABI entry points: argument validation on the host, rotation sign mask, split geometry, and
// the kernel launches.  Nothing here allocates device memory.
#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/tq.h"
#include "tq_internal.h"

namespace {

bool bits_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 8; }

constexpr int32_t kKnownFlags = TQ_FLAG_NORM_CORRECTION | TQ_FLAG_MEAN_REMOVAL | TQ_FLAG_QJL;
constexpr uint64_t kQjlSeedXor = 0x514A4C5F534B4554ull;  // sketch signs: a second stream of the seed

void fill_signs(int D, uint64_t seed, TqSigns* s) {
  uint64_t words[2];
  tq_sign_words(D, seed, words, 2);
  s->w[0] = (uint32_t)words[0];
  s->w[1] = (uint32_t)(words[0] >> 32);
  s->w[2] = (uint32_t)words[1];
  s->w[3] = (uint32_t)(words[1] >> 32);
}

int code_bytes(int D, int bits) { return (D * bits + 7) / 8; }

// Fill a TqLayer from the public descriptor.  need_q: decode also checks num_q_heads.
int make_layer(const tq_layer_desc* d, bool need_q, TqLayer* L) {
  if (d == nullptr) return TQ_ERR_INVALID_ARG;
  if ((d->flags & ~kKnownFlags) != 0) return TQ_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return TQ_ERR_UNSUPPORTED;
  if (!bits_ok(d->k_bits) || !bits_ok(d->v_bits)) return TQ_ERR_UNSUPPORTED;
  if ((d->flags & TQ_FLAG_QJL) && d->k_bits > 4) return TQ_ERR_UNSUPPORTED;  // sketches low-bit keys
  if (d->num_kv_heads < 1 || d->block_size < 1) return TQ_ERR_INVALID_ARG;
  if (d->k_centroids == nullptr || d->k_boundaries == nullptr || d->v_centroids == nullptr ||
      d->v_boundaries == nullptr)
    return TQ_ERR_INVALID_ARG;
  const int sb = tq_slot_bytes_ex(d->head_dim, d->k_bits, d->v_bits, d->flags);
  const int stride = d->slot_stride == 0 ? sb : d->slot_stride;
  if (stride < sb || (stride & 3) != 0 || stride > 4096) return TQ_ERR_INVALID_ARG;
  if (d->num_kv_heads > 64 || d->block_size > 65536) return TQ_ERR_UNSUPPORTED;
  // one page block's bytes must fit in 31 bits (row offsets inside a block are 32-bit)
  if ((int64_t)d->block_size * d->num_kv_heads * stride > ((int64_t)1 << 31)) return TQ_ERR_UNSUPPORTED;
  int G = 1;
  if (need_q) {
    if (d->num_q_heads < 1 || d->num_q_heads % d->num_kv_heads != 0) return TQ_ERR_INVALID_ARG;
    G = d->num_q_heads / d->num_kv_heads;
    if (G > 8) return TQ_ERR_UNSUPPORTED;
  }
  L->D = d->head_dim;
  L->Hq = need_q ? d->num_q_heads : d->num_kv_heads;
  L->Hkv = d->num_kv_heads;
  L->G = G;
  L->bs = d->block_size;
  L->kb = d->k_bits;
  L->vb = d->v_bits;
  L->stride = stride;
  L->slot_bytes = sb;
  L->kcode_bytes = code_bytes(d->head_dim, d->k_bits);
  L->vcode_bytes = code_bytes(d->head_dim, d->v_bits);
  L->norm_corr = (d->flags & TQ_FLAG_NORM_CORRECTION) != 0;
  L->mean = (d->flags & TQ_FLAG_MEAN_REMOVAL) != 0;
  L->qjl = (d->flags & TQ_FLAG_QJL) != 0;
  L->kqjl = L->kcode_bytes + 4 + 4 * L->mean;
  L->kreg = L->kqjl + (L->qjl ? d->head_dim / 8 + 4 : 0);
  fill_signs(d->head_dim, d->rht_seed, &L->signs);
  fill_signs(d->head_dim, d->rht_seed ^ kQjlSeedXor, &L->signs2);
  L->kc = d->k_centroids;
  L->kt = d->k_boundaries;
  L->vc = d->v_centroids;
  L->vt = d->v_boundaries;
  return TQ_OK;
}

}  // namespace

extern "C" int32_t tq_slot_bytes(int32_t D, int32_t k_bits, int32_t v_bits) {
  return tq_slot_bytes_ex(D, k_bits, v_bits, 0);
}

extern "C" int32_t tq_slot_bytes_ex(int32_t D, int32_t k_bits, int32_t v_bits, int32_t flags) {
  if (D < 1 || D > 65536 || k_bits < 1 || k_bits > 8 || v_bits < 1 || v_bits > 8)
    return TQ_ERR_INVALID_ARG;
  if ((flags & ~kKnownFlags) != 0) return TQ_ERR_INVALID_ARG;
  if ((flags & TQ_FLAG_QJL) && D % 8 != 0) return TQ_ERR_INVALID_ARG;
  const int tail = (flags & TQ_FLAG_MEAN_REMOVAL) ? 8 : 4;  // norm (and mean) per region
  const int sketch = (flags & TQ_FLAG_QJL) ? D / 8 + 4 : 0;  // key residual bits and norm
  return (code_bytes(D, k_bits) + tail + sketch) + (code_bytes(D, v_bits) + tail);
}

extern "C" int tq_quantize_append(const tq_layer_desc* layer, const void* k, const void* v,
                                  const int64_t* slot_mapping, int64_t n_tok, void* pages,
                                  int64_t num_blocks, tq_stream_t stream) {
  TqLayer L;
  const int st = make_layer(layer, false, &L);
  if (st != TQ_OK) return st;
  if (n_tok < 0 || num_blocks < 0) return TQ_ERR_INVALID_ARG;
  if (n_tok == 0) return TQ_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr || pages == nullptr)
    return TQ_ERR_INVALID_ARG;
  if (n_tok > (int64_t)1 << 40) return TQ_ERR_INVALID_ARG;
  return tq_launch_quantize(L, k, v, slot_mapping, n_tok, pages, stream) == 0 ? TQ_OK : TQ_ERR_HIP;
}

extern "C" size_t tq_decode_workspace_bytes(const tq_layer_desc* layer, int32_t num_seqs,
                                            int32_t max_seq_len) {
  TqLayer L;
  if (make_layer(layer, true, &L) != TQ_OK || num_seqs < 0 || max_seq_len < 0) return 0;
  return tq_decode_ws_bytes(L, num_seqs, tq_decode_split(L, num_seqs, max_seq_len));
}

// The split grid (packed splits of every sequence and kv head, plus the fp16-row chunks) must fit
// the kernels' 32-bit workgroup arithmetic.
static bool grid_fits(const TqLayer& L, int32_t num_seqs, const TqSplit& sp) {
  const int64_t units = (int64_t)num_seqs * sp.max_split + 8;
  // the block kernel counts the batch's runs, plus a fixed cost per sequence, in 32 bits
  if (sp.max_runs > 0 && (int64_t)num_seqs * (sp.max_runs + kTqUnitCostRuns) > INT32_MAX) return false;
  return units * L.Hkv + (int64_t)num_seqs * L.Hkv * 16 <= INT32_MAX;
}

// workspace == NULL with noalloc: the library's static array of the current device.
static int paged_decode(const tq_layer_desc* layer, const void* q, const void* pages,
                        int64_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                        const void* sink_k, const void* sink_v, int32_t n_sink, const void* win_k,
                        const void* win_v, const int32_t* win_lens, int32_t win_cap, float scale,
                        float* out, void* workspace, size_t workspace_bytes, tq_stream_t stream,
                        bool noalloc = false, const TqAppend* app = nullptr) {
  TqLayer L;
  const int st = make_layer(layer, true, &L);
  if (st != TQ_OK) return st;
  if (num_seqs < 0 || max_seq_len < 0 || n_sink < 0 || max_blocks_per_seq < 0 || num_blocks < 0 ||
      win_cap < 0)
    return TQ_ERR_INVALID_ARG;
  if (num_seqs > 65535) return TQ_ERR_UNSUPPORTED;
  if (n_sink > TQ_MAX_SINKS || win_cap > TQ_MAX_WINDOW) return TQ_ERR_UNSUPPORTED;
  if (num_seqs == 0) return TQ_OK;
  if (q == nullptr || out == nullptr || seq_lens == nullptr || (workspace == nullptr && !noalloc))
    return TQ_ERR_INVALID_ARG;
  // positions below n_sink come from the sink arrays: a batch of sink tokens only needs no pages
  if (max_seq_len > n_sink && (pages == nullptr || block_tables == nullptr))
    return TQ_ERR_INVALID_ARG;
  if (max_seq_len > n_sink && (int64_t)max_blocks_per_seq * L.bs < (int64_t)max_seq_len)
    return TQ_ERR_INVALID_ARG;
  if (n_sink > 0 && (sink_k == nullptr || sink_v == nullptr)) return TQ_ERR_INVALID_ARG;
  if (win_cap > 0 && (win_k == nullptr || win_v == nullptr || win_lens == nullptr))
    return TQ_ERR_INVALID_ARG;
  if (!(scale > 0.0f)) scale = (float)(1.0 / std::sqrt((double)L.D));
  if (!std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  const TqSplit sp = tq_decode_split(L, num_seqs, max_seq_len);
  if (!grid_fits(L, num_seqs, sp)) return TQ_ERR_UNSUPPORTED;
  if (noalloc) {
    if (tq_decode_ws_bytes_for(L, num_seqs, sp, n_sink, win_cap) > TQ_NOALLOC_WORKSPACE_BYTES)
      return TQ_ERR_NOALLOC_LIMIT;
    if (tq_noalloc_workspace(&workspace) != 0) return TQ_ERR_HIP;
  } else if (workspace_bytes < tq_decode_ws_bytes(L, num_seqs, sp)) {
    return TQ_ERR_WORKSPACE;
  }
  return tq_launch_decode(L, q, pages, block_tables, max_blocks_per_seq, seq_lens, num_seqs, sp,
                          sink_k, sink_v, n_sink, win_k, win_v, win_lens, win_cap, scale, out,
                          workspace, stream, 1, 0, 0, app) == 0
             ? TQ_OK
             : TQ_ERR_HIP;
}

extern "C" int tq_paged_decode_attention_append(const tq_layer_desc* layer, const void* q,
                                                const void* k_new, const void* v_new, void* pages,
                                                int64_t num_blocks, const int32_t* block_tables,
                                                int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                int32_t num_seqs, int32_t max_seq_len, float scale,
                                                float* out, void* workspace, size_t workspace_bytes,
                                                tq_stream_t stream) {
  TqLayer L;
  const int st = make_layer(layer, true, &L);
  if (st != TQ_OK) return st;
  if (!tq_decode_append_format(L)) return TQ_ERR_UNSUPPORTED;
  if (num_seqs > TQ_APPEND_MAX_SEQS) return TQ_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (k_new == nullptr || v_new == nullptr || pages == nullptr || block_tables == nullptr))
    return TQ_ERR_INVALID_ARG;
  const TqAppend app{k_new, v_new, pages};
  return paged_decode(layer, q, pages, num_blocks, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                      max_seq_len, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0, scale, out,
                      workspace, workspace_bytes, stream, false, &app);
}

extern "C" int tq_paged_decode_attention(const tq_layer_desc* layer, const void* q,
                                         const void* pages, int64_t num_blocks,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t num_seqs,
                                         int32_t max_seq_len, const void* sink_k,
                                         const void* sink_v, int32_t n_sink, float scale,
                                         float* out, void* workspace, size_t workspace_bytes,
                                         tq_stream_t stream) {
  return paged_decode(layer, q, pages, num_blocks, block_tables, max_blocks_per_seq, seq_lens,
                      num_seqs, max_seq_len, sink_k, sink_v, n_sink, nullptr, nullptr, nullptr, 0,
                      scale, out, workspace, workspace_bytes, stream);
}

extern "C" int tq_paged_decode_attention_noalloc(const tq_layer_desc* layer, const void* q,
                                                 const void* pages, int64_t num_blocks,
                                                 const int32_t* block_tables,
                                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                 int32_t num_seqs, int32_t max_seq_len,
                                                 const void* sink_k, const void* sink_v,
                                                 int32_t n_sink, float scale, float* out,
                                                 tq_stream_t stream) {
  return paged_decode(layer, q, pages, num_blocks, block_tables, max_blocks_per_seq, seq_lens,
                      num_seqs, max_seq_len, sink_k, sink_v, n_sink, nullptr, nullptr, nullptr, 0,
                      scale, out, nullptr, 0, stream, true);
}

extern "C" int tq_paged_decode_attention_window(
    const tq_layer_desc* layer, const void* q, const void* pages, int64_t num_blocks,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    int32_t num_seqs, int32_t max_seq_len, const void* sink_k, const void* sink_v, int32_t n_sink,
    const void* win_k, const void* win_v, const int32_t* win_lens, int32_t win_cap, float scale,
    float* out, void* workspace, size_t workspace_bytes, tq_stream_t stream) {
  return paged_decode(layer, q, pages, num_blocks, block_tables, max_blocks_per_seq, seq_lens,
                      num_seqs, max_seq_len, sink_k, sink_v, n_sink, win_k, win_v, win_lens,
                      win_cap, scale, out, workspace, workspace_bytes, stream);
}

// Queries per launch of the multi-query decode: up to 8 kernel heads per kv head.
static int queries_per_launch(const TqLayer& L) { return L.G >= 8 ? 1 : 8 / L.G; }

// The layer as one launch of the multi-query decode sees it: the queries q0 .. q0 + count - 1 as
// count * G heads per kv head.
static TqLayer multi_group(const TqLayer& L, int32_t n_queries, int q0) {
  const int per = queries_per_launch(L);
  TqLayer Lg = L;
  Lg.G = L.G * (n_queries - q0 < per ? n_queries - q0 : per);
  return Lg;
}

// Workspace of the multi-query decode: the largest of its launches' (each launch chooses its own
// kernel and split for its head count; they reuse the workspace in stream order).
static size_t multi_ws_bytes(const TqLayer& L, int32_t num_seqs, int32_t max_seq_len, int32_t n_queries) {
  size_t need = 0;
  for (int q0 = 0; q0 < n_queries; q0 += queries_per_launch(L)) {
    const TqLayer Lg = multi_group(L, n_queries, q0);
    const size_t b = tq_decode_ws_bytes(Lg, num_seqs, tq_decode_split(Lg, num_seqs, max_seq_len));
    if (b > need) need = b;
  }
  return need;
}

extern "C" size_t tq_decode_multi_workspace_bytes(const tq_layer_desc* layer, int32_t num_seqs,
                                                  int32_t max_seq_len, int32_t n_queries) {
  TqLayer L;
  if (make_layer(layer, true, &L) != TQ_OK || num_seqs < 0 || max_seq_len < 0 || n_queries < 1 ||
      n_queries > TQ_MAX_QUERIES)
    return 0;
  return multi_ws_bytes(L, num_seqs, max_seq_len, n_queries);
}

extern "C" int tq_paged_decode_attention_multi(
    const tq_layer_desc* layer, const void* q, int32_t n_queries, const void* pages,
    int64_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len, const void* sink_k,
    const void* sink_v, int32_t n_sink, float scale, float* out, void* workspace,
    size_t workspace_bytes, tq_stream_t stream) {
  TqLayer L;
  const int st = make_layer(layer, true, &L);
  if (st != TQ_OK) return st;
  if (n_queries < 1) return TQ_ERR_INVALID_ARG;
  if (n_queries > TQ_MAX_QUERIES) return TQ_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_seq_len < 0 || n_sink < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return TQ_ERR_INVALID_ARG;
  if (num_seqs > 65535) return TQ_ERR_UNSUPPORTED;
  if (n_sink > TQ_MAX_SINKS) return TQ_ERR_UNSUPPORTED;
  if (num_seqs == 0) return TQ_OK;
  if (q == nullptr || out == nullptr || seq_lens == nullptr || workspace == nullptr)
    return TQ_ERR_INVALID_ARG;
  // positions below n_sink come from the sink arrays: a batch of sink tokens only needs no pages
  if (max_seq_len > n_sink && (pages == nullptr || block_tables == nullptr))
    return TQ_ERR_INVALID_ARG;
  if (max_seq_len > n_sink && (int64_t)max_blocks_per_seq * L.bs < (int64_t)max_seq_len)
    return TQ_ERR_INVALID_ARG;
  if (n_sink > 0 && (sink_k == nullptr || sink_v == nullptr)) return TQ_ERR_INVALID_ARG;
  if (!(scale > 0.0f)) scale = (float)(1.0 / std::sqrt((double)L.D));
  if (!std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  const int per = queries_per_launch(L);
  for (int q0 = 0; q0 < n_queries; q0 += per) {
    const TqLayer Lg = multi_group(L, n_queries, q0);
    if (!grid_fits(Lg, num_seqs, tq_decode_split(Lg, num_seqs, max_seq_len))) return TQ_ERR_UNSUPPORTED;
  }
  if (workspace_bytes < multi_ws_bytes(L, num_seqs, max_seq_len, n_queries)) return TQ_ERR_WORKSPACE;
  // each group of queries is one split + merge launch pair; the pair after it reuses the
  // workspace in stream order
  for (int q0 = 0; q0 < n_queries; q0 += per) {
    const TqLayer Lg = multi_group(L, n_queries, q0);
    const TqSplit sp = tq_decode_split(Lg, num_seqs, max_seq_len);
    if (tq_launch_decode(Lg, q, pages, block_tables, max_blocks_per_seq, seq_lens, num_seqs, sp,
                         sink_k, sink_v, n_sink, nullptr, nullptr, nullptr, 0, scale, out,
                         workspace, stream, n_queries, q0, L.G) != 0)
      return TQ_ERR_HIP;
  }
  return TQ_OK;
}

extern "C" int tq_dequantize_rows(const tq_layer_desc* layer, const void* pages, int64_t num_blocks,
                                  const int64_t* slots, int64_t n, float* k_out, float* v_out,
                                  tq_stream_t stream) {
  TqLayer L;
  const int st = make_layer(layer, false, &L);
  if (st != TQ_OK) return st;
  if (n < 0 || num_blocks < 0) return TQ_ERR_INVALID_ARG;
  if (n == 0) return TQ_OK;
  if (n > ((int64_t)1 << 35) / L.Hkv) return TQ_ERR_UNSUPPORTED;  // one workgroup per 16 or 32 rows
  if (pages == nullptr || slots == nullptr || k_out == nullptr || v_out == nullptr)
    return TQ_ERR_INVALID_ARG;
  return tq_launch_dequant(L, pages, slots, n, k_out, v_out, stream) == 0 ? TQ_OK : TQ_ERR_HIP;
}

extern "C" const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported head_dim, bit width or size";
    case TQ_ERR_WORKSPACE: return "decode workspace too small";
    case TQ_ERR_HIP: return "HIP runtime error while enqueueing";
    case TQ_ERR_NO_CONVERGENCE: return "Lloyd-Max solver did not converge";
    case TQ_ERR_NOALLOC_LIMIT: return "sizes need more than the library's static decode workspace";
    default: return "unknown status";
  }
}
