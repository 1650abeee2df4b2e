/*
 * dit_timing.h -- kernel timing hook for benchmarks, exported by the
 * instrumented build libdit_probe.so only (the product library keeps no
 * timing state).
 *
 * dit_time_next_launch(start, stop) registers two HIP events (created by the
 * caller, e.g. with hipEventCreate) for the calling thread.  The next
 * epilogue or probe call into libdit_probe.so made on that thread that
 * launches a kernel does so
 * with hipExtLaunchKernelGGL, so the dispatch itself records `start` when
 * the kernel begins and `stop` when it ends; hipEventElapsedTime(start,
 * stop) is then the kernel's own duration, without the dispatch overhead
 * that separately recorded events would include.  The registration is used
 * by one launch and then cleared; a call rejected by its guards, or one
 * with nothing to launch, leaves it pending.  Passing two NULL events clears
 * it.  Always returns DIT_OK.
 */
#ifndef DIT_TIMING_H
#define DIT_TIMING_H

#include "dit.h"

#ifdef __cplusplus
extern "C" {
#endif

dit_status_t dit_time_next_launch(hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif
#endif /* DIT_TIMING_H */
