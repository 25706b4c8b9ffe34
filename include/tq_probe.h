/*
 * tq_probe.h — diagnostics of libtq (not part of the method's calls in tq.h).
 *
 * HBM streaming ceilings of the access patterns the kernels use, measured with the compute taken
 * out, so a kernel's achieved bandwidth can be set against what the same pattern can reach.
 */
#ifndef TQ_PROBE_H_
#define TQ_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef TQ_STREAM_T_DEFINED
#define TQ_STREAM_T_DEFINED
typedef struct ihipStream_t* tq_stream_t; /* a hipStream_t; NULL = the default stream */
#endif

/*
 * Reads n_blocks blocks of block_bytes bytes each from src (device) in the order order[0 ..
 * n_blocks) (device, block ids; NULL = 0, 1, 2, ...), in units of blocks_per_unit consecutive
 * entries, one unit per workgroup of 8 waves at a time (up to 1024 workgroups), each block as
 * whole 1 KB pieces.  With dst (device) given, also writes block_bytes / write_div bytes per
 * block (rounded down to 16) to dst at offset i * that size for the i-th block of the order, so
 * reads and writes stream at write_div : 1.  dst must hold n_blocks times that size.
 *   block_bytes: a multiple of 1024, at most 32768.
 * Enqueues one kernel on stream.  Returns 0, -1 for an invalid argument, -4 for a HIP error.
 * Contract violations (a block id out of range, buffers too small) are undefined behaviour.
 */
int tq_probe_stream(const void* src, int64_t n_blocks, int32_t block_bytes, const int32_t* order,
                    int32_t blocks_per_unit, void* dst, int32_t write_div, tq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H_ */
