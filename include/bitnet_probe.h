/* Measurement probes of libbitnet.so: the achievable ceilings of the two
 * resources the BitLinear forward is bound by, measured on the device the path
 * runs on.  They are not part of the method: a decode GEMV at M = 1 is bound by
 * the HBM stream of the packed weights (pages: chenxutan.com sec. 1 and sec.
 * 5.5, decoding reads every weight once per token), the prefill contraction by
 * the int8 matrix cores (sec. 3.1, the linear over the quantized operands).
 * Both calls enqueue one kernel on `stream` (a hipStream_t, NULL for the null
 * stream) and return a bitnet_status (see bitnet.h).  Timing is the caller's. */
#ifndef BITNET_PROBE_H
#define BITNET_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "bitnet.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of buf (device, 16-byte aligned, bytes % 16 == 0, bytes <
 * 2^40) once, with 16-byte non-temporal loads, lane-linear (each wavefront load
 * instruction covers 1 KB of consecutive bytes), from a grid of `blocks`
 * workgroups of 256 threads (1 .. 65536).  The loaded data are XOR-folded per
 * thread; a thread whose fold equals `key` writes it to sink[0] (device, one
 * uint32), so the loads cannot be dropped; with random data a write is
 * practically never made.  Errors: NULL buf or sink (ERR_NULL), bad size or
 * block count (ERR_SHAPE), misaligned buf or sink (ERR_ALIGN). */
BITNET_API int bitnet_probe_stream_read(const void *buf, size_t bytes, int64_t blocks, uint32_t key,
                                        uint32_t *sink, void *stream);

/* Run v_mfma_i32_16x16x64_i8 back to back from registers only: `blocks`
 * workgroups (1 .. 65536) of 8 wavefronts, each wavefront `iters` (1 .. 2^24)
 * rounds over 8 independent accumulators.  The operands derive from `key`; a
 * lane whose folded accumulators equal `key` writes to sink[0] (device, one
 * uint32).  Errors as above. */
BITNET_API int bitnet_probe_mfma_i8(int64_t blocks, int64_t iters, uint32_t key, uint32_t *sink, void *stream);

/* int8 operations (2 per multiply-add) of one bitnet_probe_mfma_i8 launch. */
BITNET_API double bitnet_probe_mfma_i8_ops(int64_t blocks, int64_t iters);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_PROBE_H */
