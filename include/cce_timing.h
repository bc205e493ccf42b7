/*
 * libcce benchmark timing hook (host only).
 *
 * This is the one piece of process-wide state in libcce, kept apart from the computation's
 * interface (cce.h) on purpose: a benchmark starts it, runs the calls it wants to time, and
 * stops it.  While it is off (the default) the calls of cce.h record nothing and keep no state.
 * It is NOT thread safe: start, use and stop it from one host thread, with no other thread
 * calling libcce meanwhile.
 */
#ifndef LIBCCE_CCE_TIMING_H
#define LIBCCE_CCE_TIMING_H

#include <stdint.h>

#include "cce.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel kinds, for per-kernel timing. */
typedef enum {
  CCE_KERNEL_FWD_LSE = 0,     /* logit tiles + online log-sum-exp partials     (2 N V D flops)   */
  CCE_KERNEL_FWD_FINISH = 1,  /* partial merge, target gather-dot, loss                          */
  CCE_KERNEL_BWD_G = 2,       /* logit recompute, softmax - onehot, filter of the first block    */
  CCE_KERNEL_BWD_FUSED = 3,   /* per (token block, vocabulary chunk) pair: dE and dC of the pair
                                 (4 Nc Vc D) with the recompute of the next pair (2 Nc' Vc' D)  */
  CCE_KERNEL_AUX = 4,         /* small helpers (statistics init, mean, zero fill, conversion)    */
  CCE_KERNEL_KINDS = 5
} cce_kernel_kind;

/* cce_timing_begin starts recording a HIP event pair around each of the next launches (at
 * most max_launches) of every kernel kind whose bit is set in kind_mask, on the stream the
 * kernel is launched on.  cce_timing_end waits for the recorded events, writes the summed
 * durations in milliseconds and the launch counts per kind into ms[CCE_KERNEL_KINDS] and
 * launches[CCE_KERNEL_KINDS] (host arrays), releases the events and stops recording.
 * Returns CCE_ERR_HIP if an event call fails, CCE_ERR_INVALID_ARGUMENT for max_launches < 1
 * or NULL outputs. */
cce_status cce_timing_begin(uint32_t kind_mask, int32_t max_launches);
cce_status cce_timing_end(float* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* LIBCCE_CCE_TIMING_H */
