/*
 * sffn_diag.h -- diagnostics of libsffn.so for benchmarks (not needed to run the
 * FFN): a read-bandwidth probe and per-launch timing of a path's main kernel.
 * Same conventions as sffn.h (device pointers, asynchronous calls, status
 * codes); these entry points do none of the FFN's arithmetic.
 */
#ifndef SFFN_DIAG_H
#define SFFN_DIAG_H

#include "sffn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Diagnostics for benchmarks: reads `bytes` (a multiple of 16, 16-byte aligned
 * device memory) once with the non-temporal 16-byte loads the decode kernels
 * use for weights, `workgroups` x 256 threads with 8 loads in flight each, and
 * writes one xor of the data per workgroup to out (device, `workgroups` words),
 * so that the read is the whole work: its time gives the HBM read ceiling for
 * that access policy.  Asynchronous on `stream`.  SFFN_ERR_INVALID_ARG for a
 * null pointer, a misaligned buffer or size, or workgroups outside 1..65536.
 */
sffn_status sffn_read_probe(const void *buf, size_t bytes, int32_t workgroups, uint32_t *out, void *stream);

/*
 * The same read with a chosen access pattern, to bound what one launch of a
 * given size can read:
 *  workgroups   1..65536
 *  threads      256, 512 or 1024 per workgroup
 *  pattern      0: grid-stride 16-byte words (the grid sweeps the buffer together);
 *               1: workgroup b reads one contiguous block of ceil(bytes / 16 / workgroups)
 *               words (the batch-1 decode kernel's pattern: each workgroup owns consecutive rows)
 *  in_flight    16-byte loads issued per thread before the first is used: 4, 8 or 16
 *  nontemporal  1: the non-temporal cache policy of the weight streams, 0: the default policy
 * out receives one xor per workgroup.  SFFN_ERR_INVALID_ARG for a null pointer, a
 * misaligned buffer or size, or a configuration outside those values.
 */
typedef struct sffn_probe_cfg {
    int32_t workgroups;
    int32_t threads;
    int32_t pattern;
    int32_t in_flight;
    int32_t nontemporal;
} sffn_probe_cfg;

sffn_status sffn_read_probe_cfg(const void *buf, size_t bytes, const sffn_probe_cfg *cfg, uint32_t *out,
                                void *stream);

/*
 * Latency of isolated row reads (the L of a latency x bandwidth merge rule):
 * one wave reads n rows of row_bytes (16..1024, a multiple of 16) at the device
 * byte offsets offsets[0..n), each read completed before the next is issued.
 * out (device, n + 2 values): out[i] = core clock cycles of read i; out[n] = core
 * cycles of the whole loop and out[n + 1] = ticks of the 100 MHz reference clock
 * over it (their ratio is the core clock).  Offsets past the buffer read its last
 * row.  SFFN_ERR_INVALID_ARG for a null pointer, n < 1, a bad row size, a buffer
 * smaller than a row or misaligned.
 */
sffn_status sffn_read_latency_probe(const void *buf, size_t bytes, int32_t row_bytes, const uint64_t *offsets,
                                    int32_t n, unsigned long long *out, void *stream);

/*
 * Diagnostics for benchmarks: arm per-launch timing of the path's main kernel
 * (the decode gate/selection kernel, the prefill gate-up GEMM).  The next n
 * sffn_forward calls on this handle launch that kernel with begin_events[i] /
 * end_events[i] (hipEvent_t, created by the caller with timing enabled) as its
 * dispatch start / stop events (hipExtLaunchKernel), so the pair brackets the
 * kernel's own execution; later calls record nothing.  The
 * arrays are host memory and must stay valid until those n calls are made.
 * n = 0 disarms.  Not thread-safe: do not arm a handle used by two threads.
 * layer = NULL arms the same timing, process-wide, for the entry points that
 * take no handle (sffn_expert_select and its one kernel, sffn_read_probe_cfg).
 */
sffn_status sffn_set_kernel_timer(sffn_t layer, void *const *begin_events, void *const *end_events,
                                  int32_t n);

/*
 * Which of the two paths of the token selection (sffn_select with a TOKENS
 * policy) made the last selection on this scratch: copies 1 (the exact-mass
 * radix select, taken when every partial sum of the scores is exact in fp64)
 * or 2 (the sort of all scores) into *path (device, one int32), asynchronously
 * on `stream`.  Meaningful only after such a selection.  SFFN_ERR_INVALID_ARG
 * for a null pointer or a layer without the PREFILL layout,
 * SFFN_ERR_WORKSPACE for a scratch smaller than the layer's.
 */
sffn_status sffn_token_select_path(sffn_t layer, const void *scratch, size_t scratch_bytes, int32_t *path,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_DIAG_H */
