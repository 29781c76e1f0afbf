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
 * Diagnostics for benchmarks: arm per-launch timing of the path's main kernel
 * (the decode gate/selection kernel, the prefill gate-up GEMM).  The next n
 * sffn_forward calls on this handle launch that kernel with begin_events[i] /
 * end_events[i] (hipEvent_t, created by the caller with timing enabled) as its
 * dispatch start / stop events (hipExtLaunchKernel), so the pair brackets the
 * kernel's own execution; later calls record nothing.  The
 * arrays are host memory and must stay valid until those n calls are made.
 * n = 0 disarms.  Not thread-safe: do not arm a handle used by two threads.
 * layer = NULL arms the same timing, process-wide, for the entry points that
 * take no handle (sffn_expert_select and its one kernel).
 */
sffn_status sffn_set_kernel_timer(sffn_t layer, void *const *begin_events, void *const *end_events,
                                  int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_DIAG_H */
