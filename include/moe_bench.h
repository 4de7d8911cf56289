/*
 * moe_bench.h -- measurement entry points of libmoe_layout.so.
 *
 * Not part of the method: these serve the benchmark and the traffic-counter
 * calibration.  The method's entry points are declared in moe_layout.h,
 * whose conventions (device pointers, stream order, MOE_* status codes)
 * apply here too.
 */
#ifndef MOE_BENCH_H
#define MOE_BENCH_H

#include "moe_layout.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Plain device copy of `bytes` (a multiple of 16; 16-byte aligned pointers),
 * one 16-byte chunk per thread: the kernel of known traffic that HBM byte
 * counters are calibrated on, and the achievable-bandwidth ceiling beside
 * the spec peak.  MOE_ERR_INVALID_ARG for a NULL pointer, MOE_ERR_SHAPE for
 * a size that is not whole chunks, MOE_ERR_ALIGNMENT for a misaligned one. */
int moe_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* Kernel timing hook.  The next kernel that a row call on this handle
 * launches (moe_dispatch, moe_combine, moe_combine_bwd, moe_dispatch_bwd or
 * a staged call; the first kernel of a call that has two) goes through
 * hipExtLaunchKernel: `stop` is bound to that kernel's completion and
 * `start`, when not NULL, is recorded just before it, so that their elapsed
 * time is the kernel's own execution, without the launch latency that
 * events recorded around the call include.  Both cost GPU time: on MI355X a
 * start marker adds about 3 us and a bound stop leaves the queue idle for
 * about 4.5 us before the next kernel (kernel-trace timestamps), so timed
 * loops that report throughput should not carry them.  One-shot: the launch
 * consumes them; both NULL disarms.  The events belong to the caller, were
 * created on the call's device, and must stay alive until the call's stream
 * has passed them.  For eager launches (not for graph capture).  Returns
 * MOE_ERR_INVALID_ARG for a bad handle, or a start without a stop.        */
int moe_time_next_kernel(moe_handle_t h, hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif
#endif /* MOE_BENCH_H */
