/*
 * fa_testing.h -- a test hook of libfa.so, outside the public ABI (include/fa.h).
 *
 * fa_testing_fwd_capped -- fa_fwd (window = 0) or fa_fwd_window (window >= 1,
 * causal != 0) with a cap on the workgroups of the persistent bf16 prefill
 * grid at d = 128.  That kernel runs one workgroup per slot that fits on the
 * device, each working through a list of (query block, head, batch) items; a
 * small cap makes every workgroup run many items in a row, which the parity
 * tests use to reach the item-switch code at sizes the oracle checks whole.
 * The cap is a per-call argument: the library keeps no setting between calls.
 * Results do not depend on it.
 *   max_workgroups 0 = no cap, >= 1 = at most that many workgroups;
 *                  < 0: FA_ERR_INVALID_ARGUMENT.
 *   window         0 = no window (causal as given), >= 1 = sliding window
 *                  (causal must be non-zero); < 0: FA_ERR_INVALID_ARGUMENT.
 *   clock_stamps   NULL, or 64 u64 of device memory (8-byte aligned) for a
 *                  clock record at d = 128 (a separate instantiation of the
 *                  kernel, the product one has no such code): workgroups 0-7 (one per
 *                  XCD) write, at stamps[8 g + 0 .. 2], the shader-cycle
 *                  counter (s_memtime), the 100 MHz real-time counter
 *                  (s_memrealtime) and the XCC id as they start, and at
 *                  stamps[8 g + 3 .. 4] the two counters as they finish.
 *                  Shader cycles over ticks times 100 MHz is the clock the
 *                  workgroup ran at.  At d = 64 nothing is written.
 * Other arguments, layouts and errors as fa_fwd.
 */
#ifndef FA_TESTING_H
#define FA_TESTING_H

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

fa_status_t fa_testing_fwd_capped(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int B, int H, int H_kv, int N_q, int N_k, int d, float scale, int causal,
                                  int window, int max_workgroups, unsigned long long* clock_stamps,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_TESTING_H */
