/*
 * rn_instrument.h — instrumentation entry point of librownorm.so for measurement
 * harnesses.  Not part of the product ABI (include/rownorm.h): no library behaviour
 * depends on it, and its state is per calling thread.
 */
#ifndef RN_INSTRUMENT_H
#define RN_INSTRUMENT_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* While `start` and `stop` are not NULL, every launch of the chosen kernel family made
 * by the CALLING THREAD records its own start and end times into them
 * (hipExtLaunchKernel events, taken by the dispatch itself): kernel 0 = forward
 * kernels, 1 = the backward's first kernel (dx and the partial rows of dW / dB).  Pass
 * NULLs to stop.  The setting is thread-local: other threads' calls are untouched.
 * Returns 0, or -2 for another kernel number. */
int rn_set_timing_events(int kernel, hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif
#endif /* RN_INSTRUMENT_H */
