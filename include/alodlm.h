/*
 * alodlm.h -- C ABI of the ALoDLM adaptively looped denoising step on MI355X (gfx950).
 *
 * The operation is one denoising step of an adaptively looped diffusion LM,
 * as described on the page "ALoDLM: Adaptively Looped Diffusion Language
 * Models" (summary of arXiv 2610.04198), sections "Core method" and
 * "Method step details" (Algorithm 1, Eq. 3):
 *
 *   h0 = Prelude(x_t) over the block rows; U = masked positions; a = 0; C = {}
 *   for s = 1..K:
 *     h~ = Core(h)                       (shared weights; prefix K/V at depth min(s, d_j))
 *     r  = RMSNorm_final(Coda(h~))
 *     for i in U: H_i = entropy(softmax(W_lm r_i)), tok_i = argmax, lambda_i = sigmoid(w_g.r_i + b_g),
 *                 a_i = a_i + (1 - a_i) lambda_i
 *     commit B = {i in U : H_i <= tau_ent}; U -= B; C += B
 *     Eq. 3: h_i = Emb(tok_i) for every i not in U, h_i = h~_i otherwise
 *     stop if U is empty, or mean_{i in U} a_i >= tau_halt, or s = K
 *   if C is empty: commit the unresolved position of lowest entropy (forced progress)
 *
 * The prefix is held in a depth-aware KV cache (same page, sections
 * "Background" and "Limitations"): Prelude and Coda layers keep one K/V set,
 * every Core layer keeps one set per loop depth 1..k_max, i.e.
 * n_pre + n_core * k_max + n_coda slots (84 for the 8B split at K = 4), or
 * only depths 1..cache_depths of the Core under depth eviction.
 *
 * Conventions for every entry point:
 *   - "device" pointers are HIP device memory on the context's device,
 *     "host" pointers are ordinary host memory.  Row-major layouts.
 *   - Nothing is allocated on the device.  Weights and the workspace are
 *     BORROWED: the caller keeps them alive and unmodified until
 *     alodlm_destroy().  The context owns only host-side metadata.
 *   - Return 0 (ALODLM_OK) on success or a negative ALODLM_E* code; on
 *     error alodlm_last_error() describes it.  Arguments are validated before
 *     any device work is enqueued, so an EINVAL call has no device effect.
 *   - All device work runs on the stream given to alodlm_create().  A context
 *     is not thread-safe; use one context per stream.
 *   - Debugging: with ALODLM_DEBUG_SYNC=1 in the environment when the context
 *     is created, the library synchronises its stream after every layer call
 *     and every readout / commit group and checks for a HIP error there; the
 *     first failure is returned (ALODLM_EHIP) by the entry point that ran it,
 *     and alodlm_last_error() names the group ("layer 12: ...", "readout of
 *     loop 2: ...").  Off by default (the step then synchronises once per loop).
 */
#ifndef ALODLM_H
#define ALODLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef ALODLM_API
#define ALODLM_API __attribute__((visibility("default")))
#endif

#define ALODLM_OK 0
#define ALODLM_EINVAL (-1)  /* bad argument (null pointer, size out of range, non-finite threshold) */
#define ALODLM_ESTATE (-2)  /* call out of order, e.g. a step before the prefix cache was built */
#define ALODLM_ENOMEM (-3)  /* workspace smaller than alodlm_workspace_bytes() */
#define ALODLM_EHIP (-4)    /* a HIP runtime call failed; the message names it */

#define ALODLM_DTYPE_BF16 0 /* bf16 weights, KV and GEMM inputs; fp32 accumulate, residual and heads */
#define ALODLM_DTYPE_FP32 1 /* fp32 everywhere */

/* Storage of keys and values (prefix cache and a block's own).  FP8: the OCP FP8 E4M3 format
 * (sign, 4 exponent bits with bias 7, 3 fraction bits, largest finite 448), rounded once from the
 * float32 result to nearest even, saturating; half the bytes of bf16 -- the compressed depth
 * buffers of the page "ALoDLM: Adaptively Looped Diffusion Language Models", section
 * "Limitations".  FP8 needs the bf16 dtype and head_dim 64 or 128. */
#define ALODLM_KV_SAME 0    /* keys and values in the config dtype */
#define ALODLM_KV_FP8 2

/* Model and capacity description. */
typedef struct alodlm_config {
  int32_t vocab;        /* V */
  int32_t d_model;      /* d, multiple of 64, at most 8192 */
  int32_t n_q_heads;    /* Hq, multiple of n_kv_heads */
  int32_t n_kv_heads;   /* Hkv */
  int32_t head_dim;     /* hd: 32, 64 or 128 */
  int32_t ffn;          /* F, multiple of 64 */
  int32_t n_pre;        /* Prelude layers (0 allowed) */
  int32_t n_core;       /* Recurrent Core layers (>= 1), run once per loop with the same weights */
  int32_t n_coda;       /* Coda layers (0 allowed) */
  int32_t k_max;        /* loop cap K and number of Core depth planes in the cache, 1..16 */
  int32_t max_batch;    /* sequences per step */
  int32_t max_prefix;   /* prefix positions held per sequence */
  int32_t max_block;    /* block (window) length L, 1..64 */
  int32_t max_prefill_rows; /* rows one prefill pass may hold (>= max_prefix); 0 = max_batch * max_prefix */
  int32_t mask_id;      /* token id of [MASK], 0..V-1 */
  int32_t dtype;        /* ALODLM_DTYPE_* */
  float rms_eps;        /* RMSNorm epsilon */
  float rope_theta;     /* RoPE base */
  int32_t depth_on_demand; /* 1: the workspace also keeps the prefix's Core output
                              ([max_batch][max_prefix][d] fp32) so that alodlm_prefill_kv_depth /
                              alodlm_deepen_kv can build the cache depth by depth; 0: not */
  int32_t kv_dtype;     /* ALODLM_KV_SAME or ALODLM_KV_FP8 */
  int32_t cache_depths; /* depth eviction (summary page, section "Limitations": the memory of the
                           per-depth buffers, remedied by dropping low-value depths): the cache
                           keeps Core depths 1..cache_depths only, so every available depth is
                           clipped to it and deeper loops read the deepest kept plane (the
                           fallback rule); 0 = every depth (k_max).  0..k_max; with
                           depth_on_demand only 0 or k_max.  The prefill still runs all k_max
                           Core passes (the Coda set is built on the depth-k_max output), the
                           deeper ones in one extra scratch plane. */
  int32_t weight_row_pad; /* elements after every row of the linear weights (wqkv, wo, w_gate_up,
                           w_down, lm_head): each is stored [out][in + weight_row_pad], the pad
                           unread.  0 = dense rows; a multiple of 8 in 0..1024.  With dense
                           4096-wide bf16 rows (8 KB apart) the same column of every row a
                           matrix tile streams falls on the same memory channels; a pad staggers
                           them (measured on the step's projections and LM head). */
} alodlm_config;

/* One transformer layer (Qwen3 block).  Device pointers in the config dtype,
 * linear maps stored [out][in] with a row pitch of in + cfg.weight_row_pad elements. */
typedef struct alodlm_layer_weights {
  const void* attn_norm;  /* [d] RMSNorm gain before attention */
  const void* wqkv;       /* [(Hq + 2 Hkv) hd][d]: q rows, then k rows, then v rows */
  const void* q_norm;     /* [hd] per-head RMSNorm gain of q */
  const void* k_norm;     /* [hd] per-head RMSNorm gain of k */
  const void* wo;         /* [d][Hq hd] */
  const void* ffn_norm;   /* [d] RMSNorm gain before the FFN */
  const void* w_gate_up;  /* [2F][d]: gate rows 0..F-1, then up rows; FFN = down(silu(gate) * up) */
  const void* w_down;     /* [d][F] */
} alodlm_layer_weights;

typedef struct alodlm_weights {
  const void* embed;       /* [V][d] token embedding (also the Eq. 3 feedback rows) */
  const void* lm_head;     /* [V][d] LMHead (row pitch d + cfg.weight_row_pad), logits z = lm_head . r */
  const void* final_norm;  /* [d] RMSNorm gain producing the readout state r */
  const void* exit_w;      /* [d] ExitGate weight: lambda = sigmoid(exit_w . r + exit_b) */
  float exit_b;            /* ExitGate bias */
  const alodlm_layer_weights* layers; /* host array of n_pre + n_core + n_coda entries, in order */
} alodlm_weights;

typedef struct alodlm_ctx alodlm_ctx;

/* Bytes of device workspace alodlm_create() needs for this config (KV cache, RoPE
 * tables and step scratch).  Host only; no device work. */
ALODLM_API int alodlm_workspace_bytes(const alodlm_config* cfg, size_t* bytes);

/* Number of prefix-cache slots: n_pre + n_core * D + n_coda, D = the kept depths (cache_depths,
 * or k_max when 0).  Slot order: Prelude layers, then each Core layer's depths 1..D, then the
 * Coda layers. */
ALODLM_API int alodlm_kv_slots(const alodlm_config* cfg, int32_t* slots);

/* Creates a context.  cfg and w are copied (the layer array too); the device
 * buffers they point to are borrowed.  workspace: device buffer of ws_bytes >=
 * alodlm_workspace_bytes(), 256-byte aligned, owned by the caller.  hip_stream:
 * a hipStream_t (NULL = default stream).  Host only: no device call is made here.
 * The first entry point that enqueues device work sets the context up on the
 * stream (RoPE tables uploaded, the V padding of the cache cleared) and
 * synchronises the stream once; a HIP failure there returns ALODLM_EHIP. */
ALODLM_API int alodlm_create(const alodlm_config* cfg, const alodlm_weights* w, void* workspace, size_t ws_bytes,
                  void* hip_stream, alodlm_ctx** out);

/* Builds the depth-aware prefix cache from token ids (summary page, section
 * "Limitations": the prefill fills every loop depth).  The prefix runs causally
 * through the Prelude once, through the Core k_max times (depth d = the d-th
 * pass) and through the Coda once on the depth-k_max output.
 *   prefix_ids:  device int32 [batch][prefix_len], ids in [0, V)
 *   avail_depth: device uint8 [batch][prefix_len], deepest Core depth cached for
 *                each position (1..k_max), used as min(loop, avail) when reading;
 *                NULL = k_max everywhere.  Copied into the workspace.
 * batch <= max_batch, 0 <= prefix_len <= max_prefix.  Asynchronous. */
ALODLM_API int alodlm_prefill_kv(alodlm_ctx* ctx, int32_t batch, int32_t prefix_len, const int32_t* prefix_ids,
                      const uint8_t* avail_depth);

/* Depth-on-demand prefill (same page, section "Limitations": the first-token latency of building
 * every depth, remedied by building depth 1 first and the deeper depths only when loops need
 * them).  Builds the Core planes of depths 1..depth only and the Prelude and Coda sets, the Coda
 * on the depth-`depth` output; every position's available depth is `depth`, so steps read the
 * deeper Core planes at `depth` (the fallback rule).  Keeps the prefix's Core output for
 * alodlm_deepen_kv.  Needs cfg.depth_on_demand (else EINVAL); 1 <= depth <= k_max.
 * alodlm_prefill_kv on such a context also keeps that state (at depth k_max).  Asynchronous. */
ALODLM_API int alodlm_prefill_kv_depth(alodlm_ctx* ctx, int32_t batch, int32_t prefix_len, const int32_t* prefix_ids,
                                       int32_t depth);

/* Continues a depth-on-demand cache to a greater depth: the Core passes from the built depth + 1
 * to `depth` over the saved Core output, then the Coda set rebuilt on the deeper output; every
 * position becomes available at `depth`.  The result equals alodlm_prefill_kv_depth(.., depth).
 * ESTATE unless the cache came from alodlm_prefill_kv_depth / alodlm_prefill_kv on a
 * depth_on_demand context and has not grown since; EINVAL unless built depth < depth <= k_max.
 * Asynchronous. */
ALODLM_API int alodlm_deepen_kv(alodlm_ctx* ctx, int32_t depth);

/* Fills the prefix cache with seeded synthetic K/V instead of computing it (for
 * long-context measurements).  Element (slot, b, h, j, e) of K is draw
 * ((b*Hkv + h)*prefix_len + j)*hd + e of Philox4x32-10 stream (seed, 0x10000 + 2*slot)
 * mapped to the Irwin-Hall(4) value times k_scale (V: stream + 1, v_scale), as
 * defined in alodlm_synth.h; `slot` numbers the slots of the cache that keeps every depth (with
 * cache_depths below k_max, the kept slots take the draws they have there).  avail_depth as in
 * alodlm_prefill_kv (clipped to the kept depths).  Asynchronous. */
ALODLM_API int alodlm_prefill_kv_synthetic(alodlm_ctx* ctx, int32_t batch, int32_t prefix_len, uint32_t seed,
                                float k_scale, float v_scale, const uint8_t* avail_depth);

#define ALODLM_STEP_TEACHER_FORCED 1u /* take commits, tokens and stop loops from tf_* */
/* Sampled commits (same page, section "Method step details", Algorithm 1 step 3: a committed
 * position takes a draw y ~ p of its readout distribution).  Without this flag the committed
 * token is the argmax (greedy).  With it, the token of readout row i of sequence b at loop s is
 * the Gumbel-max draw
 *     y = argmax_v (z_v + g_v)   (lowest v on ties),   g_v = -ln(-ln u_v),
 *     u_v = (floor(x_v / 2^9) + 1/2) / 2^23,
 * where z_v is the logit (with the planted boost) and x_v is word (v mod 4) of Philox4x32-10
 * (Salmon, Moraes, Dror, Shaw, SC'11) at counter (v div 4, 64 b + i, s, sample_step) under key
 * (sample_seed mod 2^32, sample_seed div 2^32).  b is the sequence's index in the batch and i its
 * block row.  Entropy, commit test, halting and the argmax record are unchanged; a forced commit
 * takes its row's draw of the last loop.  The same (seed, step) replays the same draws. */
#define ALODLM_STEP_SAMPLE 2u

typedef struct alodlm_step_args {
  int32_t batch;              /* sequences, == the prefilled batch */
  int32_t block_len;          /* L, <= max_block */
  const int32_t* block_ids;   /* device [batch][L]: token ids, mask_id = masked (unresolved) */
  float tau_ent;              /* commit iff entropy (nats) <= tau_ent; finite */
  float tau_halt;             /* stop when mean cumulative halt of unresolved rows >= tau_halt; finite */
  int32_t k_loops;            /* loop cap for this step, 1..k_max */
  uint32_t flags;             /* ALODLM_STEP_* */
  const int32_t* boost_tok;   /* optional device [batch][L]: planted logit boost token (-1 none) */
  const float* boost_val;     /* device [batch][L], required with boost_tok: added to that logit */
  const int8_t* tf_commit_loop; /* teacher-forced only: device [batch][L], loop s (or -s forced) or 0 */
  const int32_t* tf_tokens;   /* teacher-forced only: device [batch][L], committed token ids */
  const int8_t* tf_stop_loop; /* teacher-forced only: device [batch], loop at which the sequence stops */
  uint64_t sample_seed;       /* ALODLM_STEP_SAMPLE: Philox key of the draws */
  uint32_t sample_step;       /* ALODLM_STEP_SAMPLE: fourth counter word, e.g. the index of the denoising step */
} alodlm_step_args;

typedef struct alodlm_step_out {
  int32_t* tokens;       /* device [batch][L]: committed token, block id for rows not masked, else mask_id */
  int8_t* commit_loop;   /* device [batch][L]: s if committed at loop s, -s if forced at the last loop s, 0 */
  int8_t* loops;         /* device [batch]: loops run by each sequence; 0 for a block with no masked
                            row (nothing to denoise: it commits nothing, although its rows still pass
                            through the first loop's layers with the rest of the batch) */
  /* optional per-loop records, device [k_loops][batch][L] float (NaN where not read out): */
  float* entropy;        /* H of rows unresolved at loop start */
  float* lam;            /* ExitGate lambda */
  float* halt;           /* cumulative halt a after the update */
  float* lse;            /* log-sum-exp of the logits */
  int32_t* argmax;       /* argmax token (-1 where not read out) */
  float* hidden;         /* optional device [k_loops][batch][L][d]: Core output h~ per loop (fp32) */
  int32_t n_committed;   /* host: tokens committed by the step, filled on return */
  int32_t loops_run;     /* host: largest loop count over the batch, filled on return */
  int32_t* sampled;      /* optional device [k_loops][batch][L]: the draw of each read-out row (-1 where
                            not read out); needs ALODLM_STEP_SAMPLE and the per-loop records above */
} alodlm_step_out;

/* Runs one denoising step over the prefilled batch.  Enqueues all work on the
 * context stream and synchronises that stream once per loop to read the number
 * of sequences still looping (a few bytes), so it returns after the step has
 * finished.  Idempotent: it never writes the prefix cache. */
ALODLM_API int alodlm_denoise_step(alodlm_ctx* ctx, const alodlm_step_args* args, alodlm_step_out* out);

/* Appends n_new positions to every sequence's prefix cache: a finished block joins the prefix
 * (same page, section "Method step details", Algorithm 1 step 5: committed tokens are written
 * into the sequence before the next denoising step).  The new positions run through the stack the
 * way alodlm_prefill_kv builds the cache -- Prelude once, the Core once per depth 1..k_max, the
 * Coda once on the depth-k_max output -- causally among themselves and attending to every cached
 * position as a step reads it (Core depth min(d, available depth)).  With every cached position at
 * full depth the cache equals the prefill of the longer prefix.
 *   new_ids:   device int32 [batch][n_new], ids in [0, V)
 *   avail_new: device uint8 [batch][n_new], deepest Core depth kept for the new positions, or
 *              NULL (k_max).
 * batch == the cached batch; 1 <= n_new and cached length + n_new <= max_prefix, else EINVAL;
 * before any prefill, ESTATE.  Asynchronous. */
/* With cache_depths below k_max the new positions still run all k_max Core passes, reading cached
 * positions at the deepest kept depth min(d, available depth), and keep depths 1..cache_depths. */
ALODLM_API int alodlm_extend_kv(alodlm_ctx* ctx, int32_t batch, int32_t n_new, const int32_t* new_ids,
                                const uint8_t* avail_new);

/* Outer loop of Algorithm 1 over one block (same page, section "Method step details", steps 1
 * and 5): denoising steps until no position of the block is masked, each step starting from the
 * block with the previous steps' committed tokens written in.  Every step commits at least one
 * token of every sequence that still has a masked position (forced progress) and a sequence
 * with none runs no loop, so a block of L positions takes at most L steps. */
typedef struct alodlm_block_args {
  alodlm_step_args step;  /* the first step's arguments: block_ids = the starting block; TEACHER_FORCED is
                             not allowed; with ALODLM_STEP_SAMPLE, step t (1-based) uses
                             sample_step + t - 1 */
  int32_t max_steps;      /* cap on steps, >= 0; 0 = block_len (always enough to finish) */
  int32_t append;         /* != 0: append the finished block to the cache (alodlm_extend_kv); needs
                             max_steps 0 or >= block_len and room for block_len more positions */
  int32_t deepen;         /* != 0 (depth-on-demand caches, cfg.depth_on_demand): after a step whose loop
                             count over the batch exceeds the cache's built depth, deepen the cache
                             to that loop count (alodlm_deepen_kv) before the next step -- deeper
                             depths are built only once some loop needs them */
} alodlm_block_args;

typedef struct alodlm_block_out {
  int32_t* tokens;        /* device [batch][L]: final ids (mask_id where still masked) */
  int16_t* commit_step;   /* device [batch][L]: step (1-based) that committed the position, 0 if none */
  int8_t* commit_loop;    /* device [batch][L]: that commit's loop within its step (s, or -s forced) */
  int32_t n_steps;        /* host: steps run */
  int32_t n_committed;    /* host: tokens committed over all steps */
  int32_t built_depth;    /* host: the cache's built Core depth at the end (-1 without a depth-on-demand
                             build) */
} alodlm_block_out;

/* Runs the outer loop; reads the step's commit count back once per step (alodlm_denoise_step
 * already synchronises per loop).  Returns after the last step (and the append) is enqueued. */
ALODLM_API int alodlm_denoise_block(alodlm_ctx* ctx, const alodlm_block_args* args, alodlm_block_out* out);

/* The readout half of a loop on given readout states: LMHead entropy/argmax,
 * ExitGate and cumulative halt (a = lambda at loop 1), entropy commit, forced
 * progress and the Eq. 3 embedding rows, for n_rows rows grouped into sequences of
 * group rows (all unresolved, loop cap 1).
 *   rows: device [n_rows][d] readout states r (config dtype); n_rows <= max_batch * max_block,
 *         group in 1..64 dividing n_rows, n_rows / group <= max_batch (the per-sequence state
 *         holds max_batch sequences); else ALODLM_EINVAL
 *   boost_tok/boost_val: optional device [n_rows]
 * outputs (device): entropy, lse, lam, halt [n_rows] float; argmax, tokens [n_rows] int32;
 *   commit_loop [n_rows] int8; embed_out [n_rows][d] float (Emb(tok) for committed rows, 0 else).
 * Asynchronous. */
ALODLM_API int alodlm_readout_commit(alodlm_ctx* ctx, const void* rows, int32_t n_rows, int32_t group, float tau_ent,
                          float tau_halt, const int32_t* boost_tok, const float* boost_val, float* entropy,
                          float* lse, float* lam, float* halt, int32_t* argmax, int32_t* tokens,
                          int8_t* commit_loop, float* embed_out);

/* Bytes of the fixed scratch array that alodlm_readout_commit_static uses on each device. */
#define ALODLM_STATIC_SCRATCH_BYTES (32u << 20)

/* Allocation-free variant of alodlm_readout_commit, for callers that cannot allocate device memory
 * at call time: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, same kernels and the same outputs bit for bit; it does not touch the context's
 * workspace.  Every scratch buffer (LM-head partial statistics, unresolved flags, sequence lists,
 * counters) lives in one fixed device array inside the library, ALODLM_STATIC_SCRATCH_BYTES per
 * device, held by each device the library runs on until the process ends.  A call needs
 *   16 * n_rows * ceil(V / BN)  (BN = the LM-head column tile: 192 up to 128 rows, else 256)
 *   + about 9 * n_rows + 18 * (n_rows / group) bytes (each piece rounded up to 256)
 * and returns ALODLM_EINVAL when that exceeds the array (at V = 151936 about 3500 rows fit).
 * The array of the current device (hipGetDevice) is used; its address is looked up once per device
 * on the first call there (a failure returns ALODLM_EHIP).  Calls on one device share the array,
 * which keeps the last call's contents (every entry a call reads is written by that call first):
 * calls that overlap on one device, from several streams or threads, race on it.  Makes no
 * allocation and calls no allocating routine.  Asynchronous on the context's stream. */
ALODLM_API int alodlm_readout_commit_static(alodlm_ctx* ctx, const void* rows, int32_t n_rows, int32_t group,
                                            float tau_ent, float tau_halt, const int32_t* boost_tok,
                                            const float* boost_val, float* entropy, float* lse, float* lam,
                                            float* halt, int32_t* argmax, int32_t* tokens, int8_t* commit_loop,
                                            float* embed_out);

/* Counters of the last step: layer calls launched and loops run (host). */
ALODLM_API int alodlm_last_step_stats(const alodlm_ctx* ctx, int64_t* layer_calls, int32_t* loops_run);

/* Last error message of the context (or of the last failed create when ctx is NULL). */
ALODLM_API const char* alodlm_last_error(const alodlm_ctx* ctx);

/* Releases the host-side context.  Frees nothing it did not allocate. */
ALODLM_API void alodlm_destroy(alodlm_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif /* ALODLM_H */
