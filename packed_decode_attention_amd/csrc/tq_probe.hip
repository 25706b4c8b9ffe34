// Diagnostic kernel (not part of the method): the HBM streaming rate of the access pattern the
// block decode kernel uses, with the compute taken out, and of a read stream with a write stream
// beside it (the bulk quantize-append moves about four bytes in for one out).  It gives the
// ceilings the decode and append kernels are measured against.
//
// Work: n_blocks blocks of block_bytes (a multiple of 1 KB, at most 32 KB), taken in the order
// `order` gives (NULL: in place order), in units of per_unit consecutive order entries.  A
// persistent workgroup of 8 waves takes units in turn; wave w of a workgroup reads blocks w, w + 8,
// ... of its unit, each as block_bytes / 1024 loads of 16 bytes per lane (whole cache lines), all
// in flight together.  With a write stream, each wave then writes block_bytes / write_div bytes of
// data derived from the block (so the loads stay live) to dst at the block's place in order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeWaves = 8;
constexpr int kMaxKb = 32;

__global__ __launch_bounds__(64 * kProbeWaves) void tq_probe_stream_kernel(
    const uint8_t* __restrict__ src, int64_t n_blocks, int block_bytes, const int32_t* __restrict__ order,
    int per_unit, int64_t n_units, uint8_t* __restrict__ dst, int write_bytes) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nk = block_bytes >> 10;
  for (int64_t unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    const int64_t b0 = unit * per_unit;
    const int64_t b1 = b0 + per_unit < n_blocks ? b0 + per_unit : n_blocks;
    for (int64_t i = b0 + w; i < b1; i += kProbeWaves) {
      const int64_t blk = order != nullptr ? (int64_t)order[i] : i;
      const u32x4* p = reinterpret_cast<const u32x4*>(src + blk * block_bytes) + lane;
      u32x4 x[kMaxKb];
#pragma unroll
      for (int k = 0; k < kMaxKb; ++k) x[k] = k < nk ? p[64 * k] : u32x4{0u, 0u, 0u, 0u};
      u32x4 acc = x[0];
#pragma unroll
      for (int k = 1; k < kMaxKb; ++k) acc ^= x[k];
      if (dst != nullptr) {
        u32x4* q = reinterpret_cast<u32x4*>(dst + i * (int64_t)write_bytes);
        for (int off = lane; off < write_bytes / 16; off += 64) q[off] = acc;
      } else {
        asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));  // the loads stay live
      }
    }
  }
}

}  // namespace

extern "C" int tq_probe_stream(const void* src, int64_t n_blocks, int32_t block_bytes, const int32_t* order,
                               int32_t blocks_per_unit, void* dst, int32_t write_div, tq_stream_t stream) {
  if (src == nullptr || n_blocks < 0 || block_bytes <= 0 || block_bytes % 1024 != 0 ||
      block_bytes > kMaxKb * 1024 || blocks_per_unit <= 0 || (dst != nullptr && write_div <= 0))
    return -1;
  if (n_blocks == 0) return 0;
  const int write_bytes = dst != nullptr ? (block_bytes / write_div) & ~15 : 0;
  const int64_t n_units = (n_blocks + blocks_per_unit - 1) / blocks_per_unit;
  const int grid = n_units < 1024 ? (int)n_units : 1024;
  hipLaunchKernelGGL(tq_probe_stream_kernel, dim3(grid), dim3(64 * kProbeWaves), 0, (hipStream_t)stream,
                     (const uint8_t*)src, n_blocks, (int)block_bytes, order, (int)blocks_per_unit, n_units,
                     (uint8_t*)dst, write_bytes);
  return (int)hipGetLastError() == 0 ? 0 : -4;
}
