/*
 * alodlm_synth.h -- device fill of seeded synthetic tensors (workload generation, not the method).
 *
 * Large synthetic inputs (8B-shape weights, long-context K/V) are generated on
 * the device instead of crossing PCIe.  Each element is a pure function of
 * (seed, tensor id, element index) through Philox4x32-10 (Salmon, Moraes,
 * Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11):
 *   block n: counter (n mod 2^32, n div 2^32, 0, 0), key (seed, tensor)
 *   element i uses block i/2, words (x0, x1) if i is even, (x2, x3) if odd;
 *   z = sum of the four 16-bit halves of those words - 131070 (Irwin-Hall of order 4);
 *   value = fp32(z) * scale (one IEEE fp32 multiply), then for bf16 output
 *   rounded to nearest even.  With scale == 0 every element is `offset`.
 * The host generator of the test harness implements the same definition
 * independently; both are checked against each other element for element.
 */
#ifndef ALODLM_SYNTH_H
#define ALODLM_SYNTH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fills n elements of dst (device, dtype ALODLM_DTYPE_BF16 or _FP32) with elements
 * start .. start+n-1 of stream (seed, tensor) scaled by `scale`, or with the
 * constant `offset` when scale == 0.  Asynchronous on hip_stream.
 * Returns 0, or -1 for a null pointer / bad dtype, -4 if the launch failed. */
__attribute__((visibility("default"))) int alodlm_synth_fill(void* dst, int32_t dtype, uint64_t start, uint64_t n, uint32_t seed, uint32_t tensor,
                      float scale, float offset, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* ALODLM_SYNTH_H */
