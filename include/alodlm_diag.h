/*
 * alodlm_diag.h -- kernel-level entry points for unit tests and kernel timing.
 *
 * Not part of the method's interface: these expose the library's GEMM dispatcher
 * (the same tiles, split-K and epilogues the denoising step launches) on caller
 * buffers, so each kernel can be checked against plain arithmetic and timed at the
 * step's real shapes.  Device pointers, row-major; nothing is allocated.
 */
#ifndef ALODLM_DIAG_H
#define ALODLM_DIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ALODLM_DIAG_STORE 0  /* C[M][N] = A . B^T (fp32) */
#define ALODLM_DIAG_RESID 1  /* C[M][N] += A . B^T (fp32) */
#define ALODLM_DIAG_SWIGLU 3 /* B = [2F][K] (gate rows, then up rows); act[M][F] = silu(A.Bg^T) * (A.Bu^T) */
/* Readout statistics of the logits z = A.B^T over the N columns, the LM-head kernel of the
 * step: C[M][2] = {entropy of softmax(z), log-sum-exp of z} (fp32) and act = int32 [M]
 * argmax (lowest column among equal maxima).  scratch holds the per-column-tile partial
 * statistics: 4 * M * ceil(N / 64) floats cover every tile.  Matrix-core path only. */
#define ALODLM_DIAG_SOFTSTAT 2

/* bf16 A [M][K], B [N][K] (N = 2F for SWIGLU).  scratch: device fp32 buffer of
 * scratch_floats for split-K partials (force_splits > 1 needs splits*M*N floats).
 * force_splits: 0 = the dispatcher's choice.  force_generic != 0 runs the vector-ALU
 * kernel instead of the matrix-core one.  force_tile: -1 = the dispatcher's tile choice, else a
 * tile index of the matrix-core kernel (out of range = the dispatcher's choice).  Asynchronous.
 * Returns 0 or -1 (bad arguments, checked before any launch), -4 (launch failed). */
__attribute__((visibility("default"))) int alodlm_diag_gemm(int32_t epi, int32_t M, int32_t N, int32_t K,
                                                            const void* A, const void* B, float* C, void* act,
                                                            float* scratch, size_t scratch_floats,
                                                            int32_t force_splits, int32_t force_generic,
                                                            int32_t force_tile, void* hip_stream);

/* The matrix-core dispatcher's choice for a GEMM of M x N x K with epilogue epi (ALODLM_DIAG_*),
 * given scratch_floats of split-K scratch (the step has max_batch * max_block * max(2F, qkv) * 8):
 * tile index, split-K factor and the kernel instantiation's name as rocprofv3 reports it
 * (NUL-terminated, truncated to name_len).  For the readout epilogue (epi 2) the LM head of the
 * library's readouts: when its columns run as two launches (a 256-row readout over a vocabulary
 * whose 256-column tiles leave a last round of the compute units at most half full), both
 * instantiations with their column ranges, and *tile is the first.  Host only.  Returns 0, or -1
 * for a shape the matrix cores do not take. */
__attribute__((visibility("default"))) int alodlm_diag_gemm_choice(int32_t epi, int32_t M, int32_t N, int32_t K,
                                                                   size_t scratch_floats, int32_t* tile,
                                                                   int32_t* splits, char* name, size_t name_len);

/* Gumbel-max draws of the logits z = A.B^T (bf16 A [M][K], B [N][K]) through the step's LM-head
 * kernel: tok[m] = argmax_n (z[m][n] + g), g the Gumbel noise of ALODLM_STEP_SAMPLE in alodlm.h
 * with counter (n div 4, row_key[m], c2, c3) and key (seed mod 2^32, seed div 2^32).  row_key:
 * device int32 [M]; tok: device int32 [M].  scratch: device floats, at least 6 * M * ceil(N / 64)
 * + 3 * M.  force_generic, force_tile as in alodlm_diag_gemm.  Asynchronous.  Returns 0, -1 (bad
 * arguments, checked before any launch) or -4 (launch failed). */
__attribute__((visibility("default"))) int alodlm_diag_readout_sample(int32_t M, int32_t N, int32_t K, const void* A,
                                                                      const void* B, const int32_t* row_key,
                                                                      uint64_t seed, uint32_t c2, uint32_t c3,
                                                                      int32_t* tok, float* scratch,
                                                                      size_t scratch_floats, int32_t force_generic,
                                                                      int32_t force_tile, void* hip_stream);

/* Copies prefix-cache rows back for inspection: K and V of cache slot `slot`, sequence b,
 * positions j0 .. j0+n-1, every kv head, into dst_k / dst_v (device, config dtype,
 * [Hkv][n][hd]; the slot numbering of alodlm_kv_slots).  After a prefill the Core depth slot of
 * depth p holds position j at depth min(p, available depth of j): the values a loop-p step reads.
 * With fp8 K/V the copies are the stored E4M3 bytes.  Asynchronous on the context
 * stream.  Returns 0, -1 (bad arguments), -4 (launch failed). */
__attribute__((visibility("default"))) int alodlm_diag_read_kv(const struct alodlm_ctx* ctx, int32_t slot, int32_t b,
                                                               int32_t j0, int32_t n, void* dst_k, void* dst_v);

/* Byte offset, within the workspace, of an internal activation buffer, for inspection after a
 * call: "h" (fp32 residual rows), "xn" (normalised rows, row pitch d + 64), "attn" (attention output), "q",
 * "qkv" (fp32 projection), "act" (SwiGLU output), "r" (readout rows).  -1 if unknown. */
__attribute__((visibility("default"))) int64_t alodlm_diag_buffer_offset(const struct alodlm_ctx* ctx,
                                                                         const char* name);

/* Kernel classes timed by alodlm_diag_timing_*. */
#define ALODLM_K_GEMM_GATE_UP 0 /* FFN gate/up GEMM with the fused SwiGLU epilogue */
#define ALODLM_K_GEMM_QKV 1
#define ALODLM_K_GEMM_O 2       /* attention output projection + residual */
#define ALODLM_K_GEMM_DOWN 3    /* FFN down projection + residual */
#define ALODLM_K_ATTENTION 4    /* block attention over the depth-aware prefix cache */
#define ALODLM_K_LM_HEAD 5      /* LM-head readout GEMM + softmax-statistics merge */
#define ALODLM_K_NORM_ROPE 6    /* RMSNorms, q/k norm + RoPE, ExitGate */
#define ALODLM_K_CONTROL 7      /* commit rule, list build, Eq. 3 reset, boosts, state init */
#define ALODLM_K_CLASSES 8

struct alodlm_ctx;
/* enable != 0: every later denoising step brackets each kernel class with HIP events on the
 * context stream and accumulates their durations; enable == 0 stops and clears the counters. */
__attribute__((visibility("default"))) int alodlm_diag_timing_enable(struct alodlm_ctx* ctx, int32_t enable);
/* Accumulated milliseconds and launch count of a class since timing was enabled. */
__attribute__((visibility("default"))) int alodlm_diag_timing_read(const struct alodlm_ctx* ctx, int32_t kernel_class,
                                                                   double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* ALODLM_DIAG_H */
