/*
 * lmhead_probes.h -- measurement probes, in a library of their own
 * (liblmhead_probes.so) beside the projection's (liblmhead.so).
 *
 * Not part of the projection: two plain kernels whose rates give the HBM read
 * bandwidth and the bf16 MFMA throughput this part sustains in practice, so
 * that a caller (bench.py) can report the projection's rates as fractions of
 * the practical ceilings next to the published peaks (HBM 8 TB/s, dense bf16
 * MFMA 2.5 PFLOP/s). The conventions of lmhead.h apply: device pointers, work
 * enqueued on `stream` (a hipStream_t as void*, NULL = default stream),
 * arguments checked on the host before anything is launched, and nothing
 * allocated or synchronised; time the calls with events on that stream.
 */
#ifndef LMHEAD_PROBES_H
#define LMHEAD_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include "lmhead.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Work-groups of 256 threads the HBM probe launches (4 per compute unit). A
 * `sink` must hold lmhead_probe_grid() * 256 elements; it is written only
 * when `flag` is non-zero (callers pass 0: the flag exists so the compiler
 * keeps the work). */
int64_t lmhead_probe_grid(void);

/* Reads `bytes` of device memory at `buf` once: each of the
 * lmhead_probe_grid() work-groups streams one contiguous segment, 4 KB per
 * step across its lanes, eight steps in flight.
 *   buf    device pointer, 16-byte aligned; bytes a multiple of 16 (0: no launch)
 *   flag   0, or non-zero to store each thread's xor of the data in `sink`
 *   sink   device pointer (see lmhead_probe_grid); must not be NULL
 * Returns LMHEAD_OK, LMHEAD_ERR_INVALID (NULL pointer, misaligned buf, bytes
 * not a multiple of 16, or a segment of 4 GB or more) or LMHEAD_ERR_DEVICE
 * (launch failure). */
lmhead_status lmhead_probe_hbm_read(const void *buf, size_t bytes, int flag, uint32_t *sink,
                                    void *stream);

/* Runs two work-groups of four waves per compute unit (two waves per SIMD),
 * each wave `iters` rounds of 16 independent v_mfma_f32_16x16x32_bf16 on
 * register operands whose bf16 values are near +-1 with varied mantissas.
 *   iters  > 0
 *   flag   as above; sink: float, lmhead_probe_grid() * 256 elements
 *   flops  host pointer or NULL: receives the floating-point operations the
 *          launch performs (2 * 16 * 16 * 32 per MFMA)
 * Returns LMHEAD_OK, LMHEAD_ERR_INVALID or LMHEAD_ERR_DEVICE. */
lmhead_status lmhead_probe_mfma_bf16(int64_t iters, int flag, float *sink, void *stream,
                                     double *flops);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_PROBES_H */
