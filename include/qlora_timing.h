/*
 * qlora_timing.h -- the timing aid of libqlora_timed.so, a build of libqlora
 * for benchmarks and profilers only.  It exports everything qlora.h declares
 * (same kernels, same results) plus the call below; libqlora.so itself does
 * not export it and keeps no state between calls.
 */
#ifndef QLORA_TIMING_H
#define QLORA_TIMING_H

#include "qlora.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The next launch of this library's weight kernel -- the one kernel of a
 * call that reads the packed weights: the first quantization pass, the
 * dequantization, the weight-streaming forward (M <= 16) or the fused
 * dequant-GEMM (forward or input gradient) -- is bracketed by
 * hipEventRecord(start_event) right before it and hipEventRecord(stop_event)
 * right after it, on the stream of that call; the request is then cleared.
 * Events are hipEvent_t handles owned by the caller; NULL, NULL clears a
 * pending request.  Process-wide and not thread-safe.
 */
int qlora_time_next_weight_kernel(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_TIMING_H */
