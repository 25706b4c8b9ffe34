// Host-side driver of libtq's C ABI for sanitizer builds (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only; the kernels are not run).  Exercises the
// codebook solver, the sign vector, the size queries and every call's argument validation with
// host buffers and null device pointers: each call must return a status, never touch memory it
// was not given, and leave no undefined behaviour behind.  Exit status 0 when every expectation
// holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../include/tq.h"
#include "../include/tq_probe.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "expectation failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static tq_layer_desc layer(int D, int hq, int hkv, int bs, int kb, int vb, int flags, const float* c) {
  tq_layer_desc d;
  std::memset(&d, 0, sizeof d);
  d.head_dim = D;
  d.num_q_heads = hq;
  d.num_kv_heads = hkv;
  d.block_size = bs;
  d.k_bits = kb;
  d.v_bits = vb;
  d.slot_stride = 0;
  d.flags = flags;
  d.rht_seed = 0;
  d.k_centroids = d.v_centroids = c;
  d.k_boundaries = d.v_boundaries = c;
  return d;
}

int main() {
  // codebooks: every family, head dimension and width the kernels use, plus the extremes
  for (int family = 0; family < 2; ++family)
    for (int D : {2, 3, 64, 128, 4096})
      for (int bits = 1; bits <= 8; ++bits) {
        std::vector<float> c(1u << bits), b((1u << bits) - 1);
        std::vector<double> c64(1u << bits), b64((1u << bits) - 1);
        double mse = -1.0;
        const int st = tq_build_codebook(D, bits, family, c.data(), b.data(), c64.data(), b64.data(), &mse);
        EXPECT(st == 0 || st == -2 || st == -5);  // -2: the Beta law at D = 2 is unbounded
        if (st == 0) {
          EXPECT(mse > 0.0 && std::isfinite(mse));
          for (size_t i = 1; i < c.size(); ++i) EXPECT(c[i - 1] < c[i]);
          if (!b.empty()) EXPECT(b[b.size() / 2] == 0.0f);
        }
      }
  {
    float c[16], b[15];
    EXPECT(tq_build_codebook(1, 4, 0, c, b, nullptr, nullptr, nullptr) < 0);
    EXPECT(tq_build_codebook(128, 0, 0, c, b, nullptr, nullptr, nullptr) < 0);
    EXPECT(tq_build_codebook(128, 9, 0, c, b, nullptr, nullptr, nullptr) < 0);
    EXPECT(tq_build_codebook(128, 4, 7, c, b, nullptr, nullptr, nullptr) < 0);
    EXPECT(tq_build_codebook(128, 4, 0, nullptr, b, nullptr, nullptr, nullptr) < 0);
  }
  // sign vectors
  for (int D : {8, 64, 128, 1000}) {
    std::vector<int8_t> s(D);
    EXPECT(tq_rht_signs(D, 0x1234u, s.data()) == 0);
    for (int8_t x : s) EXPECT(x == 1 || x == -1);
  }
  EXPECT(tq_rht_signs(0, 1, nullptr) < 0);
  // slot sizes
  for (int D : {64, 128})
    for (int kb : {2, 3, 4, 8})
      for (int vb : {2, 3, 4, 8})
        for (int flags = 0; flags < 8; ++flags) {
          const int32_t n = tq_slot_bytes_ex(D, kb, vb, flags);
          if (flags == 0) EXPECT(n == tq_slot_bytes(D, kb, vb));
          EXPECT(n > 0 || n < 0);
        }
  EXPECT(tq_slot_bytes(128, 5, 4) == (80 + 4) + (64 + 4));  // the page formula, any width 1..8
  EXPECT(tq_slot_bytes(128, 0, 4) < 0);
  EXPECT(tq_slot_bytes(128, 4, 9) < 0);
  // size queries and argument validation (null device pointers: nothing may be enqueued)
  float cb[256] = {0};
  tq_layer_desc good = layer(128, 32, 8, 16, 4, 4, 0, cb);
  EXPECT(tq_decode_workspace_bytes(&good, 16, 32769) > 0);
  EXPECT(tq_decode_workspace_bytes(&good, 0, 0) == 0 || tq_decode_workspace_bytes(&good, 0, 0) > 0);
  EXPECT(tq_decode_multi_workspace_bytes(&good, 16, 1000, 0) == 0);
  EXPECT(tq_decode_multi_workspace_bytes(&good, 16, 1000, 2) > 0);
  tq_layer_desc bad[] = {layer(96, 32, 8, 16, 4, 4, 0, cb), layer(128, 30, 8, 16, 4, 4, 0, cb),
                         layer(128, 32, 8, 0, 4, 4, 0, cb), layer(128, 32, 8, 16, 5, 4, 0, cb),
                         layer(128, 32, 0, 16, 4, 4, 0, cb), layer(128, 32, 8, 16, 4, 4, 64, cb),
                         layer(128, 32, 8, 16, 4, 4, 0, nullptr)};
  for (const tq_layer_desc& d : bad) {
    EXPECT(tq_quantize_append(&d, nullptr, nullptr, nullptr, 4, nullptr, 1, nullptr) < 0);
    EXPECT(tq_paged_decode_attention(&d, nullptr, nullptr, 1, nullptr, 1, nullptr, 1, 16, nullptr, nullptr,
                                     0, 0.0f, nullptr, nullptr, 0, nullptr) < 0);
    EXPECT(tq_dequantize_rows(&d, nullptr, 1, nullptr, 1, nullptr, nullptr, nullptr) < 0);
    EXPECT(tq_decode_workspace_bytes(&d, 4, 100) == 0);
  }
  EXPECT(tq_quantize_append(nullptr, nullptr, nullptr, nullptr, 1, nullptr, 1, nullptr) < 0);
  EXPECT(tq_quantize_append(&good, nullptr, nullptr, nullptr, -1, nullptr, 1, nullptr) < 0);
  EXPECT(tq_quantize_append(&good, nullptr, nullptr, nullptr, 0, nullptr, 1, nullptr) == 0);
  EXPECT(tq_paged_decode_attention(&good, nullptr, nullptr, 1, nullptr, 1, nullptr, -1, 16, nullptr, nullptr, 0,
                                   0.0f, nullptr, nullptr, 0, nullptr) < 0);
  EXPECT(tq_paged_decode_attention(&good, nullptr, nullptr, 1, nullptr, 1, nullptr, 0, 16, nullptr, nullptr, 0,
                                   0.0f, nullptr, nullptr, 0, nullptr) == 0);
  {
    char ws[64];
    EXPECT(tq_paged_decode_attention(&good, ws, ws, 1, (const int32_t*)ws, 100000 / 16 + 1, (const int32_t*)ws, 4,
                                     100000, nullptr, nullptr, 0, 0.0f, (float*)ws, ws, sizeof ws, nullptr) == -3);
  }
  EXPECT(tq_paged_decode_attention_multi(&good, nullptr, 0, nullptr, 1, nullptr, 1, nullptr, 1, 16, nullptr,
                                         nullptr, 0, 0.0f, nullptr, nullptr, 0, nullptr) < 0);
  EXPECT(tq_probe_stream(nullptr, 1, 1024, nullptr, 1, nullptr, 0, nullptr) == -1);
  EXPECT(tq_probe_stream(cb, 1, 1000, nullptr, 1, nullptr, 0, nullptr) == -1);
  for (int s = -7; s <= 0; ++s) EXPECT(tq_status_str(s) != nullptr && tq_status_str(s)[0] != '\0');
  EXPECT(tq_status_str(-99) != nullptr);
  std::printf("host checks: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
