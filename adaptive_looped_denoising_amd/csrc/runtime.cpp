// Host runtime and C ABI of the looped denoising step: workspace plan, argument checks,
// depth-aware prefix-cache build (full, depth by depth, or grown by a finished block), the
// step driver (Prelude once, then per loop the shared Core, the Coda, the two heads, the
// commit rule, compaction and the Eq. 3 reset) and the outer loop over a block.
#include <math.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/alodlm.h"
#include "../../include/alodlm_diag.h"
#include "launch.h"
#include "common.h"

using namespace alodlm;

namespace {

thread_local std::string g_create_error;

struct Plan {
  size_t total = 0;
  // offsets (bytes) into the workspace
  size_t rope_cos, rope_sin, kcache, vcache, avail;
  size_t h, h_alt, xn, attn, qkv, q, kself, vself, gu, act;
  size_t r, lam, H, lse, tok, btok, bval, part, gpart, rkey, stok;
  size_t U, a, ro_map, ro_rows, ncommit, stop, seq_loops, act_seq0, act_seq1, src_slot, cnt;
  size_t attn_part, gemm_part;
  size_t blk_ids, blk_tok, blk_cl, blk_loops, blk_cnt;  // outer loop over a block
  size_t pstate;  // depth-on-demand: the prefix's Core output [B][P][d] fp32 (0 bytes without it)
  // sizes
  // Cache slot: K [B][Hkv][Pp][hd], V transposed [B][Hkv][hd][Pp], Pp = max_prefix rounded up to
  // 64 (a 64-key tile never leaves a V row).  Own-block V likewise [B][Hkv][hd][Lp].
  int64_t slot_elems = 0;  // elements of one cache slot: B * Hkv * Pp * hd
  int64_t Pp = 0, Lp = 0;
  int n_slots = 0, rows_step = 0, rows_max = 0, prefill_rows = 0, n_vtiles = 0, max_pos = 0;
  // depth eviction: the extra plane the Core passes of evicted depths write (-1: none), and the
  // planes allocated (n_slots, plus that one)
  int scratch_slot = -1, alloc_slots = 0;
  int attn_splits = 0;
  int av_pitch = 1;  // row pitch of the available-depth table [B][av_pitch]
  int xn_ld = 0;     // row pitch of the normalised projection inputs
  size_t gemm_part_elems = 0;
};

size_t esize(int dtype) { return dtype == ALODLM_DTYPE_BF16 ? 2 : 4; }
// Core depth planes kept in the cache (depth eviction: the first cache_depths depths)
int kept_depths(const alodlm_config& c) { return c.cache_depths > 0 ? c.cache_depths : c.k_max; }
// bytes per stored key / value element
size_t kv_esize(const alodlm_config& c) { return c.kv_dtype == ALODLM_KV_FP8 ? 1 : esize(c.dtype); }

int check_config(const alodlm_config* c, std::string* err) {
  char buf[256];
  auto bad = [&](const char* what) {
    snprintf(buf, sizeof buf, "invalid config: %s", what);
    *err = buf;
    return ALODLM_EINVAL;
  };
  if (!c) return bad("null config");
  if (c->dtype != ALODLM_DTYPE_BF16 && c->dtype != ALODLM_DTYPE_FP32) return bad("dtype");
  if (c->vocab < 2) return bad("vocab < 2");
  if (c->d_model < 64 || c->d_model % 64 || c->d_model > 8192)
    return bad("d_model must be a multiple of 64 in 64..8192");
  if (c->ffn < 64 || c->ffn % 64) return bad("ffn must be a positive multiple of 64");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 32, 64 or 128");
  if (c->n_kv_heads < 1 || c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads)
    return bad("n_q_heads must be a positive multiple of n_kv_heads");
  if (c->n_pre < 0 || c->n_coda < 0 || c->n_core < 1) return bad("layer counts");
  if (c->k_max < 1 || c->k_max > 16) return bad("k_max must be in 1..16");
  if (c->max_batch < 1 || c->max_batch > 1024) return bad("max_batch must be in 1..1024");
  if (c->max_block < 1 || c->max_block > 64) return bad("max_block must be in 1..64");
  if (c->max_prefix < 0) return bad("max_prefix < 0");
  if (c->max_prefill_rows < 0 || (c->max_prefill_rows > 0 && c->max_prefill_rows < c->max_prefix))
    return bad("max_prefill_rows must be 0 or >= max_prefix");
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return bad("mask_id outside [0, vocab)");
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps)) return bad("rms_eps");
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta)) return bad("rope_theta");
  if (c->depth_on_demand != 0 && c->depth_on_demand != 1) return bad("depth_on_demand must be 0 or 1");
  if (c->kv_dtype != ALODLM_KV_SAME && c->kv_dtype != ALODLM_KV_FP8) return bad("kv_dtype");
  if (c->cache_depths < 0 || c->cache_depths > c->k_max) return bad("cache_depths must be in 0..k_max");
  if (c->depth_on_demand && c->cache_depths > 0 && c->cache_depths < c->k_max)
    return bad("depth_on_demand needs every depth kept (cache_depths 0 or k_max)");
  if (c->kv_dtype == ALODLM_KV_FP8 && (c->dtype != ALODLM_DTYPE_BF16 || (c->head_dim != 64 && c->head_dim != 128)))
    return bad("fp8 keys and values need the bf16 dtype and head_dim 64 or 128");
  if (c->weight_row_pad < 0 || c->weight_row_pad > 1024 || c->weight_row_pad % 8)
    return bad("weight_row_pad must be a multiple of 8 in 0..1024");
  return ALODLM_OK;
}

Plan make_plan(const alodlm_config& c) {
  Plan p;
  const size_t es = esize(c.dtype);
  const int64_t B = c.max_batch, P = c.max_prefix, L = c.max_block, d = c.d_model, hd = c.head_dim;
  const int64_t Hq = c.n_q_heads, Hkv = c.n_kv_heads, F = c.ffn, V = c.vocab;
  const int64_t qkv_out = (Hq + 2 * Hkv) * hd;
  const int Dk = kept_depths(c);
  p.n_slots = c.n_pre + c.n_core * Dk + c.n_coda;
  p.scratch_slot = Dk < c.k_max ? p.n_slots : -1;
  p.alloc_slots = p.n_slots + (Dk < c.k_max ? 1 : 0);
  p.Pp = (P + 63) / 64 * 64;
  p.Lp = (L + 63) / 64 * 64;
  p.slot_elems = B * Hkv * p.Pp * hd;
  p.rows_step = (int)(B * L);
  p.prefill_rows = c.max_prefill_rows > 0 ? c.max_prefill_rows : (int)(B * P);
  p.rows_max = p.rows_step > p.prefill_rows ? p.rows_step : p.prefill_rows;
  p.n_vtiles = (int)((V + 63) / 64);
  p.max_pos = (int)(P + L);
  p.attn_splits = 16;
  const int64_t R = p.rows_max, Rs = p.rows_step;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  p.rope_cos = take(sizeof(float) * p.max_pos * (hd / 2));
  p.rope_sin = take(sizeof(float) * p.max_pos * (hd / 2));
  const size_t kes = kv_esize(c);
  p.kcache = take(kes * p.slot_elems * p.alloc_slots);
  p.vcache = take(kes * p.slot_elems * p.alloc_slots);
  p.av_pitch = P > 0 ? (int)P : 1;
  p.avail = take(B * p.av_pitch);
  p.h = take(sizeof(float) * R * d);
  p.h_alt = take(sizeof(float) * R * d);
  p.xn_ld = (int)d + 64;  // padded row pitch: the projections stream 128-byte pieces of many rows
  p.xn = take(es * R * p.xn_ld);
  p.attn = take(es * R * Hq * hd);
  p.qkv = take(sizeof(float) * R * qkv_out);
  p.q = take(es * R * Hq * hd);
  p.kself = take(kes * Rs * Hkv * hd);
  p.vself = take(kes * B * Hkv * hd * p.Lp);
  p.gu = take(sizeof(float) * R * 2 * F);
  p.act = take(es * R * F);
  p.r = take(es * Rs * d);
  p.lam = take(sizeof(float) * Rs);
  p.H = take(sizeof(float) * Rs);
  p.lse = take(sizeof(float) * Rs);
  p.tok = take(sizeof(int32_t) * Rs);
  p.btok = take(sizeof(int32_t) * Rs);
  p.bval = take(sizeof(float) * Rs);
  p.part = take(16 * Rs * (size_t)p.n_vtiles);
  p.gpart = take(8 * Rs * (size_t)p.n_vtiles);
  p.rkey = take(sizeof(int32_t) * Rs);
  p.stok = take(sizeof(int32_t) * Rs);
  p.U = take(Rs);
  p.a = take(sizeof(float) * Rs);
  p.ro_map = take(sizeof(int32_t) * Rs);
  p.ro_rows = take(sizeof(int32_t) * Rs);
  p.ncommit = take(sizeof(int32_t) * B);
  p.stop = take(B);
  p.seq_loops = take(B);
  p.act_seq0 = take(sizeof(int32_t) * B);
  p.act_seq1 = take(sizeof(int32_t) * B);
  p.src_slot = take(sizeof(int32_t) * B);
  p.cnt = take(sizeof(int32_t) * 8);
  p.attn_part = take(sizeof(float) * Rs * Hq * (size_t)p.attn_splits * (hd + 2));
  p.gemm_part_elems = (size_t)Rs * (size_t)(2 * F > qkv_out ? 2 * F : qkv_out) * 8;
  p.gemm_part = take(sizeof(float) * p.gemm_part_elems);
  p.blk_ids = take(sizeof(int32_t) * Rs);
  p.blk_tok = take(sizeof(int32_t) * Rs);
  p.blk_cl = take(Rs);
  p.blk_loops = take(B);
  p.blk_cnt = take(sizeof(int32_t) * 4);
  p.pstate = take(c.depth_on_demand ? sizeof(float) * B * P * d : 0);
  p.total = off;
  return p;
}

}  // namespace

struct alodlm_ctx {
  alodlm_config cfg;
  alodlm_weights w;
  std::vector<alodlm_layer_weights> layers;
  Plan plan;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t st = nullptr;
  std::string err;
  bool dev_ready = false;  // RoPE tables uploaded and V padding cleared (first device call)
  // prefix cache state
  int cache_batch = -1, cache_prefix = -1;
  int built_depth = -1;  // depth-on-demand: Core depth the prefix state holds (-1: no state)
  int state_prefix = -1; // prefix length the saved state covers
  // stats of the last step
  int64_t layer_calls = 0;
  int32_t loops_run = 0;
  bool force_generic = false;  // diagnostics: ALODLM_FORCE_GENERIC=1 keeps bf16 on the vector-ALU kernels
  int attn_force_splits = 0;   // diagnostics: ALODLM_ATTN_SPLITS=n fixes the key splits of step attention
  int attn_force_qw = 0;       // diagnostics: ALODLM_ATTN_QW=16|32 fixes the query rows per wave
  int attn_force_ns = 0;       // diagnostics: ALODLM_ATTN_NS=2..4 fixes the LDS ring depth
  int attn_force_nw = 0;       // diagnostics: ALODLM_ATTN_NW=4|8 fixes the waves per workgroup
  int attn_force_kh = 0;       // diagnostics: ALODLM_ATTN_KH=1|2 fixes the key halves per tile
  int proj_splits[3] = {0, 0, 0};  // diagnostics: ALODLM_PROJ_SPLITS=q,o,d fixes the QKV / O / down split-K
  int proj_tiles[4] = {-1, -1, -1, -1};  // diagnostics: ALODLM_PROJ_TILES=q,o,d,gu fixes their GEMM tiles
  int lm_tile = -1;            // diagnostics: ALODLM_LM_TILE=t fixes the LM-head readout's GEMM tile (a 256 x 256 tile keeps the column ranges)
  // diagnostics: per-class kernel timing with event pairs on the context stream
  bool timing = false;
  std::vector<hipEvent_t> ev_pool;
  std::vector<int> ev_class;  // class of each recorded pair
  size_t ev_used = 0;
  double t_ms[ALODLM_K_CLASSES] = {0};
  int64_t t_n[ALODLM_K_CLASSES] = {0};

  bool in_step = false;  // timing covers denoising steps only
  void tic(int cls) {
    if (!timing || !in_step) return;
    const size_t i = ev_used * 2;
    while (ev_pool.size() < i + 2) {
      hipEvent_t e;
      hipEventCreate(&e);
      ev_pool.push_back(e);
    }
    ev_class.resize(ev_used + 1);
    ev_class[ev_used] = cls;
    hipEventRecord(ev_pool[i], st);
  }
  void toc() {
    if (!timing || !in_step) return;
    hipEventRecord(ev_pool[ev_used * 2 + 1], st);
    ++ev_used;
  }
  // After a stream synchronisation: fold the recorded pairs into the totals.
  void fold() {
    for (size_t k = 0; k < ev_used; ++k) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev_pool[2 * k], ev_pool[2 * k + 1]) == hipSuccess) {
        t_ms[ev_class[k]] += ms;
        t_n[ev_class[k]] += 1;
      }
    }
    ev_used = 0;
  }
  ~alodlm_ctx() {
    for (hipEvent_t e : ev_pool) hipEventDestroy(e);
  }

  template <typename T>
  T* at(size_t off) const {
    return (T*)(ws + off);
  }
  int fail(int code, const std::string& m) {
    err = m;
    return code;
  }
  int hip_check(const char* what) {
    if (!debug_first.empty()) {
      const std::string m = "debug sync: " + debug_first;
      debug_first.clear();
      return fail(ALODLM_EHIP, m);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ALODLM_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return ALODLM_OK;
  }
  // diagnostics: ALODLM_DEBUG_SYNC=1 synchronises the stream after every layer call and every
  // readout / commit group and checks for a HIP error there, so that a failing launch is named
  // by its group; the first failure is kept and returned by the entry point's next error check.
  bool debug_sync = false;
  std::string debug_first;
  void dbg_point(const char* what, int index) {
    if (!debug_sync || !debug_first.empty()) return;
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) debug_first = std::string(what) + " " + std::to_string(index) + ": " + hipGetErrorString(e);
  }
};

namespace {

int dt(const alodlm_ctx* c) { return c->cfg.dtype == ALODLM_DTYPE_BF16 ? DT_BF16 : DT_FP32; }

void* cache_slot(alodlm_ctx* c, bool v, int slot) {
  return c->ws + (v ? c->plan.vcache : c->plan.kcache) + kv_esize(c->cfg) * (size_t)c->plan.slot_elems * slot;
}

// storage type of keys and values (DT_FP8, or the model dtype)
int kvt(const alodlm_ctx* c) { return c->cfg.kv_dtype == ALODLM_KV_FP8 ? DT_FP8 : dt(c); }

// Stored slot of (layer, loop depth); a Core depth beyond the kept ones reads the deepest kept.
int slot_of(const alodlm_config& c, int layer, int depth) {
  const int Dk = kept_depths(c);
  if (layer < c.n_pre) return layer;
  if (layer < c.n_pre + c.n_core) return c.n_pre + (layer - c.n_pre) * Dk + ((depth < Dk ? depth : Dk) - 1);
  return c.n_pre + c.n_core * Dk + (layer - c.n_pre - c.n_core);
}

// Slot index of a stored slot in the layout that keeps every depth (the synthetic cache's streams)
int full_slot(const alodlm_config& c, int slot) {
  const int Dk = kept_depths(c);
  if (slot < c.n_pre) return slot;
  if (slot < c.n_pre + c.n_core * Dk) {
    const int ci = (slot - c.n_pre) / Dk, d = (slot - c.n_pre) % Dk;
    return c.n_pre + ci * c.k_max + d;
  }
  return slot + c.n_core * (c.k_max - Dk);
}

bool use_mfma(const alodlm_ctx* c, int K, int lda, int ldb) {
  return c->cfg.dtype == ALODLM_DTYPE_BF16 && !c->force_generic && gemm_mfma_supported(K, lda, ldb);
}

// GEMM dispatch: C = A . B^T with the given epilogue (SWIGLU: N = 2F interleaved gate/up).
// With `defer`, a split-K STORE / RESID GEMM may leave its partials unreduced in the split-K
// scratch for the consuming kernel; the return value is then the number of partials (else 1).
int gemm(alodlm_ctx* c, int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
         const int32_t* m_dev, const GemmEpi& ep, int F = 0, bool defer = false, int force_splits = 0,
         int force_tile = -1) {
  if (use_mfma(c, K, lda, ldb)) {
    return launch_gemm_mfma(epi, A, lda, B, ldb, M, N, K, m_dev, ep, F, c->at<float>(c->plan.gemm_part),
                            c->plan.gemm_part_elems, force_splits, c->st, force_tile, defer);
  }
  if (epi == EPI_SWIGLU) {  // generic path: both halves in fp32, then silu(gate) * up
    GemmEpi e;
    e.C = c->at<float>(c->plan.gu);
    e.ldc = N;
    launch_gemm_generic(dt(c), EPI_STORE, A, lda, B, ldb, M, N, K, m_dev, e, c->st);
    launch_swiglu(dt(c), e.C, M, F, ep.act, c->st);
    return 1;
  }
  launch_gemm_generic(dt(c), epi, A, lda, B, ldb, M, N, K, m_dev, ep, c->st);
  return 1;
}

// Column tiles of the LM-head softmax statistics for the path a readout of M rows takes.
int lm_tiles(const alodlm_ctx* c, int M) {
  const int d = c->cfg.d_model;
  if (!use_mfma(c, d, d, d + c->cfg.weight_row_pad)) return (c->cfg.vocab + 63) / 64;
  SoftstatPlan sp;
  gemm_mfma_softstat_plan(M, c->cfg.vocab, c->lm_tile, &sp);
  return sp.n_tiles;
}

// The LM-head GEMM with the readout-statistics epilogue over the whole vocabulary for M rows
// (rows >= *n_dev skipped): one launch, or on the matrix cores two column ranges
// (gemm_mfma_softstat_plan) whose partials sit side by side in each row's ep.n_tiles entries.
void lm_head_gemm(alodlm_ctx* c, const void* rows, int M, const int32_t* n_dev, const GemmEpi& ep) {
  const alodlm_config& g = c->cfg;
  const int d = g.d_model, ldw = d + g.weight_row_pad;
  if (!use_mfma(c, d, d, ldw)) {
    gemm(c, EPI_SOFTSTAT, rows, d, c->w.lm_head, ldw, M, g.vocab, d, n_dev, ep, 0, false, 0, c->lm_tile);
    return;
  }
  SoftstatPlan sp;
  gemm_mfma_softstat_plan(M, g.vocab, c->lm_tile, &sp);
  gemm(c, EPI_SOFTSTAT, rows, d, c->w.lm_head, ldw, M, sp.cols0, d, n_dev, ep, 0, false, 0, sp.tile0);
  if (sp.tile1 >= 0) {
    GemmEpi e2 = ep;
    e2.part = ep.part + sp.tiles0;
    if (ep.smp.part) e2.smp.part = ep.smp.part + sp.tiles0;
    e2.col0 = sp.cols0;
    const void* w1 = (const char*)c->w.lm_head + (size_t)sp.cols0 * ldw * esize(g.dtype);
    gemm(c, EPI_SOFTSTAT, rows, d, w1, ldw, M, g.vocab - sp.cols0, d, n_dev, e2, 0, false, 0, sp.tile1);
  }
}

void attention(alodlm_ctx* c, const AttnParams& p) {
  const bool kv8 = c->cfg.kv_dtype == ALODLM_KV_FP8;  // fp8 keys and values: matrix-core path only
  if (c->cfg.dtype == ALODLM_DTYPE_BF16 && (kv8 || !c->force_generic) && attn_mfma_supported(p.hd)) {
    AttnParams q = p;
    q.kv8 = kv8 ? 1 : 0;
    q.part = c->at<float>(c->plan.attn_part);
    launch_attn_mfma(q, c->plan.attn_splits, c->st, c->attn_force_splits, c->attn_force_qw, c->attn_force_ns,
                     c->attn_force_nw, c->attn_force_kh);
    return;
  }
  launch_attn_generic(dt(c), p, c->st);
}

enum Mode { STEP, PREFILL };

struct LayerCall {
  Mode mode;
  const float* x_in;
  float* x_out;
  int n_rows, rows_per_seq, pos0;
  // step: sequence map and loop; prefill: first sequence of the group and depth
  const int32_t* seq_map;
  int loop;
  int seq0, depth;
  int prefix_len;
  // chaining of the FFN down projection into the next layer: `defer` lets this layer leave its
  // split-K partials unreduced (the caller guarantees the next launch is run_layer on the same
  // rows, reading x_out as its x_in); `pend` > 1 says x_in still lacks that many partials, which
  // the attention RMSNorm adds (in place) before normalising.
  bool defer = false;
  int pend = 1;
};

// One transformer block over n_rows rows: x_out = block(x_in).  In prefill mode the rows'
// post-RoPE K/V go straight into the cache slot of (layer, depth) and attention is causal
// over them; in step mode the rows attend to the prefix cache (depth-selected for Core
// layers) plus their own block's K/V.
int run_layer(alodlm_ctx* c, int li, const LayerCall& lc) {
  const alodlm_config& g = c->cfg;
  const alodlm_layer_weights& W = c->layers[li];
  const Plan& p = c->plan;
  const int d = g.d_model, hd = g.head_dim, Hq = g.n_q_heads, Hkv = g.n_kv_heads, F = g.ffn;
  const int qkv_out = (Hq + 2 * Hkv) * hd;
  const int wp = g.weight_row_pad;  // weight rows are in + wp elements apart
  const int n = lc.n_rows;
  const size_t es = esize(g.dtype);
  (void)es;
  void* xn = c->at<void>(p.xn);
  void* attn = c->at<void>(p.attn);
  float* qkv = c->at<float>(p.qkv);
  void* q = c->at<void>(p.q);
  void* act = c->at<void>(p.act);

  const int xp = p.xn_ld;
  c->tic(ALODLM_K_NORM_ROPE);
  if (lc.pend > 1)  // finish the previous layer's down projection: x_in += its partials, in place
    launch_rmsnorm(dt(c), lc.x_in, n, d, nullptr, nullptr, W.attn_norm, g.rms_eps, xn, nullptr, 0.f, nullptr, c->st,
                   c->at<float>(p.gemm_part), lc.pend, const_cast<float*>(lc.x_in), xp);
  else
    launch_rmsnorm(dt(c), lc.x_in, n, d, nullptr, nullptr, W.attn_norm, g.rms_eps, xn, nullptr, 0.f, nullptr, c->st,
                   nullptr, 1, nullptr, xp);
  c->toc();
  GemmEpi e1;
  e1.C = qkv;
  e1.ldc = qkv_out;
  c->tic(ALODLM_K_GEMM_QKV);
  const int qkv_splits = gemm(c, EPI_STORE, xn, xp, W.wqkv, d + wp, n, qkv_out, d, nullptr, e1, 0, true, c->proj_splits[0],
                             c->proj_tiles[0]);
  c->toc();
  const float* qkv_src = qkv_splits > 1 ? c->at<float>(p.gemm_part) : qkv;

  AttnParams ap;
  ap.q = q;
  ap.out = attn;
  ap.n_rows = n;
  ap.rows_per_seq = lc.rows_per_seq;
  ap.Hq = Hq;
  ap.Hkv = Hkv;
  ap.hd = hd;
  ap.scale = 1.0f / sqrtf((float)hd);
  const int64_t Pp = p.Pp, Lp = p.Lp;
  if (lc.mode == PREFILL) {
    // rows are positions pos0 .. pos0 + rows_per_seq - 1 of each sequence: their post-RoPE K/V go
    // into the slot right after the pos0 positions already there, and they attend causally to
    // all of them (pos0 = 0 for a prefill from scratch, the cached length when a block is appended).
    // A Core pass of an evicted depth works in the scratch plane (its keys are needed only by
    // itself).
    // A Core pass of an evicted depth keeps its rows' keys in the scratch plane (from position 0)
    // and reads the positions already there from the deepest kept plane.
    const bool core_l = li >= g.n_pre && li < g.n_pre + g.n_core;
    const bool evicted = core_l && lc.depth > kept_depths(g);
    const int slot = evicted ? p.scratch_slot : slot_of(g, li, lc.depth);
    const int at = evicted ? 0 : lc.pos0;  // position of the first row in the written plane
    void* kd = cache_slot(c, false, slot);
    void* vd = cache_slot(c, true, slot);
    const int64_t kSeq = (int64_t)Hkv * Pp * hd, kHead = Pp * hd, kPos = hd;
    const int64_t vSeq = (int64_t)Hkv * hd * Pp, vHead = hd * Pp, vRow = Pp;
    const size_t es_ = kv_esize(g);
    c->tic(ALODLM_K_NORM_ROPE);
    launch_qk_norm_rope(dt(c), qkv_src, n, lc.rows_per_seq, lc.pos0, Hq, Hkv, hd, W.q_norm, W.k_norm, g.rms_eps,
                        c->at<float>(p.rope_cos), c->at<float>(p.rope_sin), q,
                        (char*)kd + (size_t)at * kPos * es_, (char*)vd + (size_t)at * es_, kSeq, kHead,
                        kPos, vSeq, vHead, vRow, lc.seq0, c->st, qkv_splits, kvt(c));
    c->toc();
    ap.n_cache = 0;
    if (evicted && lc.pos0 > 0) {
      const int ks = slot_of(g, li, kept_depths(g));
      ap.ck = (const char*)cache_slot(c, false, ks) + (size_t)lc.seq0 * kSeq * es_;
      ap.cv = (const char*)cache_slot(c, true, ks) + (size_t)lc.seq0 * vSeq * es_;
      ap.c_kSeq = kSeq;
      ap.c_kHead = kHead;
      ap.c_kPos = kPos;
      ap.c_vSeq = vSeq;
      ap.c_vHead = vHead;
      ap.c_vRow = vRow;
      ap.n_cache = lc.pos0;
    }
    ap.sk = kd;
    ap.sv = vd;
    ap.s_kSeq = kSeq;
    ap.s_kHead = kHead;
    ap.s_kPos = kPos;
    ap.s_vSeq = vSeq;
    ap.s_vHead = vHead;
    ap.s_vRow = vRow;
    ap.s_seq0 = lc.seq0;
    ap.n_self = at + lc.rows_per_seq;
    ap.causal = 1;
    ap.causal_off = at;
  } else {
    void* ks = c->at<void>(p.kself);
    void* vs = c->at<void>(p.vself);
    const int64_t kSeq = (int64_t)lc.rows_per_seq * Hkv * hd, kHead = hd, kPos = (int64_t)Hkv * hd;
    const int64_t vSeq = (int64_t)Hkv * hd * Lp, vHead = hd * Lp, vRow = Lp;
    c->tic(ALODLM_K_NORM_ROPE);
    launch_qk_norm_rope(dt(c), qkv_src, n, lc.rows_per_seq, lc.pos0, Hq, Hkv, hd, W.q_norm, W.k_norm, g.rms_eps,
                        c->at<float>(p.rope_cos), c->at<float>(p.rope_sin), q, ks, vs, kSeq, kHead, kPos, vSeq, vHead,
                        vRow, 0, c->st, qkv_splits, kvt(c));
    c->toc();
    // Core layers read the depth plane of the loop: the planes are materialised after the prefill
    // (plane s holds every position at depth min(s, available depth))
    const bool core = li >= g.n_pre && li < g.n_pre + g.n_core;
    const int slot = slot_of(g, li, core ? lc.loop : 1);
    ap.ck = cache_slot(c, false, slot);
    ap.cv = cache_slot(c, true, slot);
    ap.c_kSeq = (int64_t)Hkv * Pp * hd;
    ap.c_kHead = Pp * hd;
    ap.c_kPos = hd;
    ap.c_vSeq = (int64_t)Hkv * hd * Pp;
    ap.c_vHead = hd * Pp;
    ap.c_vRow = Pp;
    ap.n_cache = lc.prefix_len;
    ap.seq_map = lc.seq_map;
    ap.sk = ks;
    ap.sv = vs;
    ap.s_kSeq = kSeq;
    ap.s_kHead = kHead;
    ap.s_kPos = kPos;
    ap.s_vSeq = vSeq;
    ap.s_vHead = vHead;
    ap.s_vRow = vRow;
    ap.n_self = lc.rows_per_seq;
    ap.causal = 0;
  }
  c->tic(ALODLM_K_ATTENTION);
  attention(c, ap);
  c->toc();

  GemmEpi e2;
  e2.C = lc.x_out;
  e2.R = lc.x_in;
  e2.ldc = d;
  c->tic(ALODLM_K_GEMM_O);
  const int o_splits =
      gemm(c, EPI_RESID, attn, Hq * hd, W.wo, Hq * hd + wp, n, d, Hq * hd, nullptr, e2, 0, true, c->proj_splits[1],
           c->proj_tiles[1]);
  c->toc();

  // FFN RMSNorm; with deferred O-projection partials it also forms x_out = x_in + sum(partials)
  c->tic(ALODLM_K_NORM_ROPE);
  if (o_splits > 1)
    launch_rmsnorm(dt(c), lc.x_in, n, d, nullptr, nullptr, W.ffn_norm, g.rms_eps, xn, nullptr, 0.f, nullptr, c->st,
                   c->at<float>(p.gemm_part), o_splits, lc.x_out, xp);
  else
    launch_rmsnorm(dt(c), lc.x_out, n, d, nullptr, nullptr, W.ffn_norm, g.rms_eps, xn, nullptr, 0.f, nullptr,
                   c->st, nullptr, 1, nullptr, xp);
  c->toc();
  GemmEpi e3;
  e3.act = act;
  e3.ld_act = F;
  c->tic(ALODLM_K_GEMM_GATE_UP);
  gemm(c, EPI_SWIGLU, xn, xp, W.w_gate_up, d + wp, n, 2 * F, d, nullptr, e3, F, false, 0, c->proj_tiles[3]);
  c->toc();
  GemmEpi e4;
  e4.C = lc.x_out;
  e4.R = lc.x_out;
  e4.ldc = d;
  c->tic(ALODLM_K_GEMM_DOWN);
  const int down_splits = gemm(c, EPI_RESID, act, F, W.w_down, F + wp, n, d, F, nullptr, e4, 0, lc.defer, c->proj_splits[2],
                                c->proj_tiles[2]);
  c->toc();
  c->layer_calls += 1;
  c->dbg_point("layer", li);
  return down_splits;
}

// LMHead statistics of the readout rows (rows >= *n_dev skipped) then the fixed-order merge; with
// smp also the Gumbel-max draw of each row (into the stok buffer).
void readout_heads(alodlm_ctx* c, const void* rows, int n_upper, const int32_t* n_dev, const int32_t* btok,
                   const float* bval, const SampleParams* smp) {
  const alodlm_config& g = c->cfg;
  const Plan& p = c->plan;
  GemmEpi ep;
  ep.part = c->at<SoftStat>(p.part);
  ep.n_tiles = lm_tiles(c, n_upper);
  ep.btok = btok;
  ep.bval = bval;
  if (smp) {
    ep.smp = *smp;
    ep.smp.part = c->at<GStat>(p.gpart);
  }
  lm_head_gemm(c, rows, n_upper, n_dev, ep);
  launch_softstat_combine(c->at<SoftStat>(p.part), n_upper, ep.n_tiles, n_dev, c->at<float>(p.H),
                          c->at<float>(p.lse), c->at<int32_t>(p.tok), smp ? ep.smp.part : nullptr,
                          smp ? c->at<int32_t>(p.stok) : nullptr, c->st);
}

bool finite_f(float x) { return isfinite(x) != 0; }

}  // namespace

// ---------------------------------------------------------------------------------------------
extern "C" {

int alodlm_workspace_bytes(const alodlm_config* cfg, size_t* bytes) {
  std::string err;
  int rc = check_config(cfg, &err);
  if (rc) {
    g_create_error = err;
    return rc;
  }
  if (!bytes) {
    g_create_error = "null bytes pointer";
    return ALODLM_EINVAL;
  }
  *bytes = make_plan(*cfg).total;
  return ALODLM_OK;
}

int alodlm_kv_slots(const alodlm_config* cfg, int32_t* slots) {
  std::string err;
  int rc = check_config(cfg, &err);
  if (rc) {
    g_create_error = err;
    return rc;
  }
  if (!slots) return ALODLM_EINVAL;
  *slots = cfg->n_pre + cfg->n_core * kept_depths(*cfg) + cfg->n_coda;
  return ALODLM_OK;
}

int alodlm_create(const alodlm_config* cfg, const alodlm_weights* w, void* workspace, size_t ws_bytes,
                  void* hip_stream, alodlm_ctx** out) {
  std::string err;
  int rc = check_config(cfg, &err);
  if (rc) {
    g_create_error = err;
    return rc;
  }
  if (!out || !w) {
    g_create_error = "null weights or output pointer";
    return ALODLM_EINVAL;
  }
  *out = nullptr;
  const int nl = cfg->n_pre + cfg->n_core + cfg->n_coda;
  if (!w->embed || !w->lm_head || !w->final_norm || !w->exit_w || !w->layers || !finite_f(w->exit_b)) {
    g_create_error = "null weight pointer or non-finite exit_b";
    return ALODLM_EINVAL;
  }
  for (int i = 0; i < nl; ++i) {
    const alodlm_layer_weights& L = w->layers[i];
    if (!L.attn_norm || !L.wqkv || !L.q_norm || !L.k_norm || !L.wo || !L.ffn_norm || !L.w_gate_up || !L.w_down) {
      g_create_error = "null pointer in layer " + std::to_string(i);
      return ALODLM_EINVAL;
    }
  }
  if (!workspace || ((uintptr_t)workspace & 255)) {
    g_create_error = "workspace null or not 256-byte aligned";
    return ALODLM_EINVAL;
  }
  Plan plan = make_plan(*cfg);
  if (ws_bytes < plan.total) {
    g_create_error = "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(plan.total);
    return ALODLM_ENOMEM;
  }
  alodlm_ctx* c = new alodlm_ctx();
  c->cfg = *cfg;
  c->w = *w;
  c->layers.assign(w->layers, w->layers + nl);
  c->w.layers = c->layers.data();
  c->plan = plan;
  c->ws = (char*)workspace;
  c->ws_bytes = ws_bytes;
  c->st = (hipStream_t)hip_stream;
  const char* fg = getenv("ALODLM_FORCE_GENERIC");
  c->force_generic = fg && fg[0] == '1';
  if (const char* v = getenv("ALODLM_ATTN_SPLITS")) c->attn_force_splits = atoi(v);
  if (const char* v = getenv("ALODLM_ATTN_QW")) c->attn_force_qw = atoi(v);
  if (const char* v = getenv("ALODLM_ATTN_NS")) c->attn_force_ns = atoi(v);
  if (const char* v = getenv("ALODLM_ATTN_NW")) c->attn_force_nw = atoi(v);
  if (const char* v = getenv("ALODLM_ATTN_KH")) c->attn_force_kh = atoi(v);
  if (const char* v = getenv("ALODLM_DEBUG_SYNC")) c->debug_sync = v[0] == '1';
  if (const char* v = getenv("ALODLM_PROJ_SPLITS"))
    sscanf(v, "%d,%d,%d", &c->proj_splits[0], &c->proj_splits[1], &c->proj_splits[2]);
  if (const char* v = getenv("ALODLM_PROJ_TILES"))
    sscanf(v, "%d,%d,%d,%d", &c->proj_tiles[0], &c->proj_tiles[1], &c->proj_tiles[2], &c->proj_tiles[3]);
  if (const char* v = getenv("ALODLM_LM_TILE")) c->lm_tile = atoi(v);
  *out = c;
  return ALODLM_OK;
}

namespace {
// Device set-up of a context, run by the first entry point that enqueues device work (creation
// itself touches no device, so argument checks of every entry point run without one): the RoPE
// tables, computed in double on the host (angle(pos, i) = pos * theta^(-2i/hd)), are uploaded,
// and the V cache and own-block V start at zero -- V rows are read in whole 64-key tiles whose
// masked keys get probability 0, so their padding must hold finite values (0 * NaN would poison
// the sum).  Synchronises the stream once.
int ensure_device(alodlm_ctx* c) {
  if (c->dev_ready) return ALODLM_OK;
  const alodlm_config* cfg = &c->cfg;
  const Plan& plan = c->plan;
  const int half = cfg->head_dim / 2;
  std::vector<float> cs((size_t)plan.max_pos * half), sn((size_t)plan.max_pos * half);
  for (int pos = 0; pos < plan.max_pos; ++pos)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)pos * pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
      cs[(size_t)pos * half + i] = (float)cos(ang);
      sn[(size_t)pos * half + i] = (float)sin(ang);
    }
  hipError_t e1 = hipMemcpyAsync(c->ws + plan.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, c->st);
  hipError_t e2 = hipMemcpyAsync(c->ws + plan.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, c->st);
  const size_t es = kv_esize(*cfg);
  if (e1 == hipSuccess) e1 = hipMemsetAsync(c->ws + plan.vcache, 0, es * plan.slot_elems * plan.alloc_slots, c->st);
  if (e1 == hipSuccess)
    e1 = hipMemsetAsync(c->ws + plan.vself, 0, es * (size_t)cfg->max_batch * cfg->n_kv_heads * cfg->head_dim * plan.Lp,
                        c->st);
  hipError_t e3 = hipStreamSynchronize(c->st);
  if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess)
    return c->fail(ALODLM_EHIP, std::string("context set-up (RoPE tables, V padding): ") +
                                    hipGetErrorString(e1 != hipSuccess ? e1 : (e2 != hipSuccess ? e2 : e3)));
  c->dev_ready = true;
  return ALODLM_OK;
}
}  // namespace

namespace {
// Fill each Core layer's higher depth planes of positions j0 .. j0+n-1 from their available depth
// (see launch_materialize_depth).
void materialize_depths(alodlm_ctx* c, int batch, int j0, int n) {
  const alodlm_config& g = c->cfg;
  const Plan& p = c->plan;
  for (int ci = 0; ci < g.n_core; ++ci) {
    const int s0 = slot_of(g, g.n_pre + ci, 1);
    launch_materialize_depth(kvt(c), cache_slot(c, false, s0), cache_slot(c, true, s0), p.slot_elems, kept_depths(g), batch,
                             g.n_kv_heads, j0, n, (int)p.Pp, g.head_dim, c->at<uint8_t>(p.avail), p.av_pitch, c->st);
  }
}
}  // namespace

namespace {
// Prefill passes over the prefix of every sequence, in groups of sequences that fit the prefill
// rows: Prelude, Core depths 1..depth (each pass writing its depth slot), Coda on the
// depth-`depth` output.  With `save`, the Core output at that depth is kept in the prefill
// state buffer (depth-on-demand).
void prefill_passes(alodlm_ctx* c, int batch, int prefix_len, const int32_t* prefix_ids, int depth, bool save) {
  const alodlm_config& g = c->cfg;
  const Plan& p = c->plan;
  const int per = p.prefill_rows / prefix_len;  // sequences per pass (>= 1: prefill_rows >= max_prefix)
  float* h = c->at<float>(p.h);
  for (int b0 = 0; b0 < batch; b0 += per) {
    const int gb = batch - b0 < per ? batch - b0 : per;
    const int n = gb * prefix_len;
    launch_embed_rows(dt(c), prefix_ids + (size_t)b0 * prefix_len, n, c->w.embed, g.d_model, g.vocab, h, c->st);
    LayerCall lc{PREFILL, h, h, n, prefix_len, 0, nullptr, 1, b0, 1, prefix_len};
    for (int li = 0; li < g.n_pre; ++li) run_layer(c, li, lc);
    for (int dpt = 1; dpt <= depth; ++dpt) {
      lc.depth = dpt;
      for (int ci = 0; ci < g.n_core; ++ci) run_layer(c, g.n_pre + ci, lc);
    }
    if (save)
      hipMemcpyAsync(c->at<float>(p.pstate) + (size_t)b0 * prefix_len * g.d_model, h,
                     sizeof(float) * (size_t)n * g.d_model, hipMemcpyDeviceToDevice, c->st);
    lc.depth = 1;
    for (int ci = 0; ci < g.n_coda; ++ci) run_layer(c, g.n_pre + g.n_core + ci, lc);
  }
}

int prefill_common(alodlm_ctx* c, int32_t batch, int32_t prefix_len, const int32_t* prefix_ids,
                   const uint8_t* avail_depth, int depth) {
  const alodlm_config& g = c->cfg;
  if (batch < 1 || batch > g.max_batch) return c->fail(ALODLM_EINVAL, "batch outside 1..max_batch");
  if (prefix_len < 0 || prefix_len > g.max_prefix) return c->fail(ALODLM_EINVAL, "prefix_len outside 0..max_prefix");
  if (prefix_len > 0 && !prefix_ids) return c->fail(ALODLM_EINVAL, "null prefix_ids");
  if (int rc0 = ensure_device(c)) return rc0;
  const Plan& p = c->plan;
  c->cache_batch = -1;
  c->built_depth = -1;
  if (depth == g.k_max)
    launch_set_avail(c->at<uint8_t>(p.avail), p.av_pitch, 0, batch, prefix_len, avail_depth, (uint8_t)g.k_max, (uint8_t)kept_depths(g), c->st);
  else
    launch_set_avail(c->at<uint8_t>(p.avail), p.av_pitch, 0, batch, prefix_len, nullptr, (uint8_t)depth, (uint8_t)kept_depths(g), c->st);
  const bool save = g.depth_on_demand != 0;
  if (prefix_len > 0) {
    prefill_passes(c, batch, prefix_len, prefix_ids, depth, save);
    materialize_depths(c, batch, 0, prefix_len);
  }
  int rc = c->hip_check("prefill launch");
  if (rc) return rc;
  c->cache_batch = batch;
  c->cache_prefix = prefix_len;
  if (save) {
    c->built_depth = depth;
    c->state_prefix = prefix_len;
  }
  return ALODLM_OK;
}
}  // namespace

int alodlm_prefill_kv(alodlm_ctx* c, int32_t batch, int32_t prefix_len, const int32_t* prefix_ids,
                      const uint8_t* avail_depth) {
  if (!c) return ALODLM_EINVAL;
  return prefill_common(c, batch, prefix_len, prefix_ids, avail_depth, c->cfg.k_max);
}

int alodlm_prefill_kv_depth(alodlm_ctx* c, int32_t batch, int32_t prefix_len, const int32_t* prefix_ids,
                            int32_t depth) {
  if (!c) return ALODLM_EINVAL;
  if (!c->cfg.depth_on_demand) return c->fail(ALODLM_EINVAL, "config without depth_on_demand");
  if (depth < 1 || depth > c->cfg.k_max) return c->fail(ALODLM_EINVAL, "depth outside 1..k_max");
  return prefill_common(c, batch, prefix_len, prefix_ids, nullptr, depth);
}

int alodlm_deepen_kv(alodlm_ctx* c, int32_t depth) {
  if (!c) return ALODLM_EINVAL;
  const alodlm_config& g = c->cfg;
  if (!g.depth_on_demand) return c->fail(ALODLM_EINVAL, "config without depth_on_demand");
  if (c->cache_batch < 0 || c->built_depth < 1 || c->cache_prefix != c->state_prefix)
    return c->fail(ALODLM_ESTATE, "deepen needs a cache built by alodlm_prefill_kv_depth and not grown since");
  if (depth <= c->built_depth || depth > g.k_max)
    return c->fail(ALODLM_EINVAL, "depth must exceed the built depth and be at most k_max");
  const Plan& p = c->plan;
  const int batch = c->cache_batch, P = c->cache_prefix, d0 = c->built_depth;
  if (P > 0) {
    const int per = p.prefill_rows / P;
    float* h = c->at<float>(p.h);
    for (int b0 = 0; b0 < batch; b0 += per) {
      const int gb = batch - b0 < per ? batch - b0 : per;
      const int n = gb * P;
      float* st_rows = c->at<float>(p.pstate) + (size_t)b0 * P * g.d_model;
      hipMemcpyAsync(h, st_rows, sizeof(float) * (size_t)n * g.d_model, hipMemcpyDeviceToDevice, c->st);
      LayerCall lc{PREFILL, h, h, n, P, 0, nullptr, 1, b0, 1, P};
      for (int dpt = d0 + 1; dpt <= depth; ++dpt) {
        lc.depth = dpt;
        for (int ci = 0; ci < g.n_core; ++ci) run_layer(c, g.n_pre + ci, lc);
      }
      hipMemcpyAsync(st_rows, h, sizeof(float) * (size_t)n * g.d_model, hipMemcpyDeviceToDevice, c->st);
      lc.depth = 1;
      for (int ci = 0; ci < g.n_coda; ++ci) run_layer(c, g.n_pre + g.n_core + ci, lc);
    }
    launch_set_avail(c->at<uint8_t>(p.avail), p.av_pitch, 0, batch, P, nullptr, (uint8_t)depth, (uint8_t)kept_depths(g), c->st);
    materialize_depths(c, batch, 0, P);
  }
  int rc = c->hip_check("deepen launch");
  if (rc) return rc;
  c->built_depth = depth;
  return ALODLM_OK;
}

int alodlm_prefill_kv_synthetic(alodlm_ctx* c, int32_t batch, int32_t prefix_len, uint32_t seed, float k_scale,
                                float v_scale, const uint8_t* avail_depth) {
  if (!c) return ALODLM_EINVAL;
  const alodlm_config& g = c->cfg;
  if (batch < 1 || batch > g.max_batch) return c->fail(ALODLM_EINVAL, "batch outside 1..max_batch");
  if (prefix_len < 0 || prefix_len > g.max_prefix) return c->fail(ALODLM_EINVAL, "prefix_len outside 0..max_prefix");
  if (!finite_f(k_scale) || !finite_f(v_scale)) return c->fail(ALODLM_EINVAL, "non-finite scale");
  if (int rc0 = ensure_device(c)) return rc0;
  const Plan& p = c->plan;
  c->cache_batch = -1;
  c->built_depth = -1;
  launch_set_avail(c->at<uint8_t>(p.avail), p.av_pitch, 0, batch, prefix_len, avail_depth, (uint8_t)g.k_max, (uint8_t)kept_depths(g), c->st);
  for (int s = 0; s < p.n_slots; ++s) {
    launch_fill_kv_synth(kvt(c), cache_slot(c, false, s), batch, g.n_kv_heads, prefix_len, (int)p.Pp, g.head_dim,
                         seed, 0x10000u + 2u * full_slot(g, s), k_scale, false, c->st);
    launch_fill_kv_synth(kvt(c), cache_slot(c, true, s), batch, g.n_kv_heads, prefix_len, (int)p.Pp, g.head_dim,
                         seed, 0x10000u + 2u * full_slot(g, s) + 1u, v_scale, true, c->st);
  }
  if (prefix_len > 0) materialize_depths(c, batch, 0, prefix_len);
  int rc = c->hip_check("synthetic prefill launch");
  if (rc) return rc;
  c->cache_batch = batch;
  c->cache_prefix = prefix_len;
  return ALODLM_OK;
}

int alodlm_extend_kv(alodlm_ctx* c, int32_t batch, int32_t n_new, const int32_t* new_ids,
                     const uint8_t* avail_new) {
  if (!c) return ALODLM_EINVAL;
  const alodlm_config& g = c->cfg;
  if (c->cache_batch < 0) return c->fail(ALODLM_ESTATE, "extend before the prefix cache was built");
  if (batch != c->cache_batch) return c->fail(ALODLM_EINVAL, "batch differs from the cached batch");
  const int P0 = c->cache_prefix;
  if (n_new < 1 || n_new > g.max_prefix - P0)
    return c->fail(ALODLM_EINVAL, "n_new outside 1 .. max_prefix - cached length");
  if (!new_ids) return c->fail(ALODLM_EINVAL, "null new_ids");
  const Plan& p = c->plan;
  const int per = p.prefill_rows / n_new;  // >= 1: prefill_rows >= max_prefix >= n_new
  float* h = c->at<float>(p.h);
  for (int b0 = 0; b0 < batch; b0 += per) {
    const int gb = batch - b0 < per ? batch - b0 : per;
    const int n = gb * n_new;
    launch_embed_rows(dt(c), new_ids + (size_t)b0 * n_new, n, c->w.embed, g.d_model, g.vocab, h, c->st);
    LayerCall lc{PREFILL, h, h, n, n_new, P0, nullptr, 1, b0, 1, P0 + n_new};
    for (int li = 0; li < g.n_pre; ++li) run_layer(c, li, lc);
    for (int dpt = 1; dpt <= g.k_max; ++dpt) {
      lc.depth = dpt;
      for (int ci = 0; ci < g.n_core; ++ci) run_layer(c, g.n_pre + ci, lc);
    }
    lc.depth = 1;
    for (int ci = 0; ci < g.n_coda; ++ci) run_layer(c, g.n_pre + g.n_core + ci, lc);
  }
  launch_set_avail(c->at<uint8_t>(p.avail), p.av_pitch, P0, batch, n_new, avail_new, (uint8_t)g.k_max, (uint8_t)kept_depths(g), c->st);
  if (avail_new) materialize_depths(c, batch, P0, n_new);
  int rc = c->hip_check("extend launch");
  if (rc) return rc;
  c->cache_prefix = P0 + n_new;
  return ALODLM_OK;
}

int alodlm_denoise_step(alodlm_ctx* c, const alodlm_step_args* a, alodlm_step_out* o) {
  if (!c) return ALODLM_EINVAL;
  if (!a || !o) return c->fail(ALODLM_EINVAL, "null args or out");
  const alodlm_config& g = c->cfg;
  const Plan& p = c->plan;
  const int B = a->batch, L = a->block_len, K = a->k_loops, d = g.d_model;
  if (c->cache_batch < 0) return c->fail(ALODLM_ESTATE, "denoise_step before the prefix cache was built");
  if (B != c->cache_batch) return c->fail(ALODLM_EINVAL, "batch differs from the prefilled batch");
  if (L < 1 || L > g.max_block) return c->fail(ALODLM_EINVAL, "block_len outside 1..max_block");
  if (K < 1 || K > g.k_max) return c->fail(ALODLM_EINVAL, "k_loops outside 1..k_max");
  if (!finite_f(a->tau_ent) || !finite_f(a->tau_halt)) return c->fail(ALODLM_EINVAL, "non-finite threshold");
  if (!a->block_ids) return c->fail(ALODLM_EINVAL, "null block_ids");
  if (a->boost_tok && !a->boost_val) return c->fail(ALODLM_EINVAL, "boost_tok without boost_val");
  const bool tf = (a->flags & ALODLM_STEP_TEACHER_FORCED) != 0;
  if (tf && (!a->tf_commit_loop || !a->tf_tokens || !a->tf_stop_loop))
    return c->fail(ALODLM_EINVAL, "teacher-forced step without tf_* arrays");
  if (!o->tokens || !o->commit_loop || !o->loops) return c->fail(ALODLM_EINVAL, "null output array");
  const bool dbg = o->entropy || o->lam || o->halt || o->lse || o->argmax;
  if (dbg && !(o->entropy && o->lam && o->halt && o->lse && o->argmax))
    return c->fail(ALODLM_EINVAL, "per-loop records must be all given or all null");
  const bool smp = (a->flags & ALODLM_STEP_SAMPLE) != 0;
  if (o->sampled && !(smp && dbg))
    return c->fail(ALODLM_EINVAL, "the sampled record needs ALODLM_STEP_SAMPLE and the other per-loop records");
  if (a->flags & ~(ALODLM_STEP_TEACHER_FORCED | ALODLM_STEP_SAMPLE)) return c->fail(ALODLM_EINVAL, "unknown flags");
  const int P = c->cache_prefix;
  hipStream_t st = c->st;
  c->layer_calls = 0;
  struct StepScope {
    alodlm_ctx* c;
    explicit StepScope(alodlm_ctx* x) : c(x) { c->in_step = true; c->ev_used = 0; }
    ~StepScope() { c->in_step = false; c->ev_used = 0; }
  } scope(c);

  uint8_t* U = c->at<uint8_t>(p.U);
  float* av = c->at<float>(p.a);
  int32_t* ncommit = c->at<int32_t>(p.ncommit);
  uint8_t* stop = c->at<uint8_t>(p.stop);
  int32_t* act[2] = {c->at<int32_t>(p.act_seq0), c->at<int32_t>(p.act_seq1)};
  int32_t* src_slot = c->at<int32_t>(p.src_slot);
  int32_t* ro_rows = c->at<int32_t>(p.ro_rows);
  int32_t* ro_map = c->at<int32_t>(p.ro_map);
  int32_t* cnt = c->at<int32_t>(p.cnt);
  float* h = c->at<float>(p.h);
  float* h_alt = c->at<float>(p.h_alt);

  if (dbg) {
    const size_t n = (size_t)K * B * L;
    hipMemsetAsync(o->entropy, 0xFF, n * 4, st);  // NaN until written
    hipMemsetAsync(o->lam, 0xFF, n * 4, st);
    hipMemsetAsync(o->halt, 0xFF, n * 4, st);
    hipMemsetAsync(o->lse, 0xFF, n * 4, st);
    hipMemsetAsync(o->argmax, 0xFF, n * 4, st);
    if (o->sampled) hipMemsetAsync(o->sampled, 0xFF, n * 4, st);  // -1 until written
  }
  launch_step_init(a->block_ids, B, L, g.mask_id, U, av, o->tokens, o->commit_loop, ncommit, stop, o->loops, act[0],
                   src_slot, st);
  launch_build_lists(B, L, B, 1, act[0], stop, U, ncommit, act[1], src_slot, ro_rows, ro_map, cnt, st);
  int cur = 1;

  // Prelude over every block row (slot t = sequence t)
  launch_embed_rows(dt(c), a->block_ids, B * L, c->w.embed, d, g.vocab, h, st);
  LayerCall lc{STEP, h, h, B * L, L, P, act[cur], 1, 0, 1, P};
  // run one layer; `chain`: the next launch is the next layer on this layer's output
  auto layer = [&](int li, bool chain) {
    lc.defer = chain;
    lc.pend = run_layer(c, li, lc);
  };
  for (int li = 0; li < g.n_pre; ++li) layer(li, true);  // the first Core layer follows the Prelude

  int nb = B;
  int32_t host_cnt[3] = {0, 0, 0};
  int loops_run = 0;
  for (int s = 1; s <= K && nb > 0; ++s) {
    loops_run = s;
    const int n = nb * L;
    lc.n_rows = n;
    lc.seq_map = act[cur];
    lc.loop = s;
    lc.x_in = h;
    lc.x_out = h;
    for (int ci = 0; ci < g.n_core; ++ci)
      layer(g.n_pre + ci, ci + 1 < g.n_core || (g.n_coda > 0 && !o->hidden));
    if (o->hidden) launch_dump_hidden(nb, L, d, B, s, act[cur], h, o->hidden, st);
    const float* gsrc = h;
    if (g.n_coda > 0) {
      lc.x_in = h;
      lc.x_out = h_alt;
      for (int ci = 0; ci < g.n_coda; ++ci) {
        layer(g.n_pre + g.n_core + ci, ci + 1 < g.n_coda);
        lc.x_in = h_alt;
      }
      gsrc = h_alt;
    }
    // readout rows r (compact), ExitGate lambda
    c->tic(ALODLM_K_NORM_ROPE);
    launch_rmsnorm(dt(c), gsrc, n, d, ro_rows, cnt + 1, c->w.final_norm, g.rms_eps, c->at<void>(p.r), c->w.exit_w,
                   c->w.exit_b, c->at<float>(p.lam), st);
    c->toc();
    // per-readout-row boosts and sampling row keys, gathered into readout order on the device
    // (row t*L+i of the compact list is sequence act[t], block row i)
    const int32_t* bt = nullptr;
    const float* bv = nullptr;
    if (a->boost_tok) {
      bt = c->at<int32_t>(p.btok);
      bv = c->at<float>(p.bval);
    }
    launch_gather_rows(ro_rows, cnt + 1, act[cur], n, L, a->boost_tok, a->boost_val, c->at<int32_t>(p.btok),
                       c->at<float>(p.bval), smp ? c->at<int32_t>(p.rkey) : nullptr, st);
    SampleParams sp;
    if (smp) {
      sp.row_key = c->at<int32_t>(p.rkey);
      sp.k0 = (uint32_t)(a->sample_seed & 0xFFFFFFFFu);
      sp.k1 = (uint32_t)(a->sample_seed >> 32);
      sp.c2 = (uint32_t)s;
      sp.c3 = a->sample_step;
    }
    // after loop 1 the host holds the exact readout row count (read back with the loop status),
    // which picks the LM-head tile; loop 1 uses the bound n
    const int n_read = (s > 1 && host_cnt[1] > 0 && host_cnt[1] <= n) ? host_cnt[1] : n;
    c->tic(ALODLM_K_LM_HEAD);
    readout_heads(c, c->at<void>(p.r), n_read, cnt + 1, bt, bv, smp ? &sp : nullptr);
    c->toc();
    c->dbg_point("readout of loop", s);
    c->tic(ALODLM_K_CONTROL);
    launch_commit(nb, s, K, L, B, a->tau_ent, a->tau_halt, act[cur], U, av, ro_map, c->at<float>(p.H),
                  c->at<int32_t>(p.tok), smp ? c->at<int32_t>(p.stok) : nullptr, c->at<float>(p.lam),
                  c->at<float>(p.lse), o->tokens, o->commit_loop, ncommit, stop, o->loops,
                  tf ? a->tf_commit_loop : nullptr, tf ? a->tf_tokens : nullptr, tf ? a->tf_stop_loop : nullptr,
                  dbg ? o->entropy : nullptr, o->lam, o->halt, o->lse, o->argmax, o->sampled, st);
    launch_build_lists(nb, L, B, 0, act[cur], stop, U, ncommit, act[cur ^ 1], src_slot, ro_rows, ro_map, cnt, st);
    launch_reset_compact(dt(c), nb, cnt, L, d, g.vocab, act[cur ^ 1], src_slot, U, o->tokens, h, c->w.embed, h_alt, st);
    c->toc();
    c->dbg_point("commit and compaction of loop", s);
    float* t = h;
    h = h_alt;
    h_alt = t;
    cur ^= 1;
    hipError_t e1 = hipMemcpyAsync(host_cnt, cnt, sizeof(host_cnt), hipMemcpyDeviceToHost, st);
    hipError_t e2 = hipStreamSynchronize(st);
    if (e1 != hipSuccess || e2 != hipSuccess)
      return c->fail(ALODLM_EHIP, std::string("loop status read: ") + hipGetErrorString(e1 != hipSuccess ? e1 : e2));
    int rc = c->hip_check("step launch");
    if (rc) return rc;
    c->fold();
    nb = host_cnt[0];
  }
  o->n_committed = host_cnt[2];
  o->loops_run = loops_run;
  c->loops_run = loops_run;
  return ALODLM_OK;
}

int alodlm_denoise_block(alodlm_ctx* c, const alodlm_block_args* a, alodlm_block_out* o) {
  if (!c) return ALODLM_EINVAL;
  if (!a || !o) return c->fail(ALODLM_EINVAL, "null args or out");
  if (!o->tokens || !o->commit_step || !o->commit_loop) return c->fail(ALODLM_EINVAL, "null output array");
  const alodlm_config& g = c->cfg;
  const Plan& p = c->plan;
  const int B = a->step.batch, L = a->step.block_len;
  if (a->step.flags & ALODLM_STEP_TEACHER_FORCED) return c->fail(ALODLM_EINVAL, "teacher forcing in the outer loop");
  if (c->cache_batch < 0) return c->fail(ALODLM_ESTATE, "denoise_block before the prefix cache was built");
  if (B != c->cache_batch) return c->fail(ALODLM_EINVAL, "batch differs from the prefilled batch");
  if (L < 1 || L > g.max_block) return c->fail(ALODLM_EINVAL, "block_len outside 1..max_block");
  if (!a->step.block_ids) return c->fail(ALODLM_EINVAL, "null block_ids");
  if (a->max_steps < 0) return c->fail(ALODLM_EINVAL, "max_steps < 0");
  const int max_steps = a->max_steps == 0 ? L : a->max_steps;
  if (a->append && (max_steps < L || L > g.max_prefix - c->cache_prefix))
    return c->fail(ALODLM_EINVAL, "append needs max_steps 0 or >= block_len and room for block_len positions");
  if (a->deepen && !g.depth_on_demand) return c->fail(ALODLM_EINVAL, "deepen needs cfg.depth_on_demand");
  hipStream_t st = c->st;
  const int n = B * L;
  int32_t* ids = c->at<int32_t>(p.blk_ids);
  int32_t* cnt = c->at<int32_t>(p.blk_cnt);
  launch_block_init(a->step.block_ids, n, g.mask_id, ids, o->commit_step, o->commit_loop, cnt, st);
  int32_t masked = 0;
  hipError_t e1 = hipMemcpyAsync(&masked, cnt, sizeof(masked), hipMemcpyDeviceToHost, st);
  hipError_t e2 = hipStreamSynchronize(st);
  if (e1 != hipSuccess || e2 != hipSuccess)
    return c->fail(ALODLM_EHIP, std::string("mask count read: ") + hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  int steps = 0, committed = 0;
  while (masked - committed > 0 && steps < max_steps) {
    ++steps;
    alodlm_step_args sa = a->step;
    sa.block_ids = ids;
    sa.sample_step = a->step.sample_step + (uint32_t)(steps - 1);
    alodlm_step_out so;
    memset(&so, 0, sizeof(so));
    so.tokens = c->at<int32_t>(p.blk_tok);
    so.commit_loop = c->at<int8_t>(p.blk_cl);
    so.loops = c->at<int8_t>(p.blk_loops);
    int rc = alodlm_denoise_step(c, &sa, &so);
    if (rc) return rc;
    launch_block_merge(n, steps, so.tokens, so.commit_loop, ids, o->commit_step, o->commit_loop, st);
    committed += so.n_committed;
    if (so.n_committed < 1) return c->fail(ALODLM_ESTATE, "internal: an outer-loop step committed nothing");
    // depth on demand: a loop ran past the built depth, so build up to that depth for the next step
    if (a->deepen && c->built_depth > 0 && c->state_prefix == c->cache_prefix && so.loops_run > c->built_depth) {
      rc = alodlm_deepen_kv(c, so.loops_run);
      if (rc) return rc;
    }
  }
  if (hipMemcpyAsync(o->tokens, ids, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return c->fail(ALODLM_EHIP, "block tokens copy");
  o->n_steps = steps;
  o->n_committed = committed;
  o->built_depth = c->built_depth;
  if (a->append) {
    int rc = alodlm_extend_kv(c, B, L, ids, nullptr);
    if (rc) return rc;
  }
  return c->hip_check("block launch");
}

}  // extern "C"

namespace {
// Scratch buffers of one readout (alodlm_readout_commit and its allocation-free variant).
struct ReadoutScratch {
  SoftStat* part;  // [n_rows][column tiles] LM-head partial statistics
  uint8_t* U;      // [n_rows] unresolved flags
  int32_t *ro_map, *ro_rows;                     // [n_rows]
  int32_t *act0, *act1, *src_slot, *ncommit;     // [sequences]
  uint8_t* stop;                                 // [sequences]
  int8_t* seq_loops;                             // [sequences]
  int32_t* cnt;                                  // [8]
};

int readout_check(alodlm_ctx* c, const void* rows, int32_t n_rows, int32_t group, float tau_ent, float tau_halt,
                  const int32_t* boost_tok, const float* boost_val, float* entropy, float* lse, float* lam, float* halt,
                  int32_t* argmax, int32_t* tokens, int8_t* commit_loop, float* embed_out) {
  const alodlm_config& g = c->cfg;
  if (!rows || !entropy || !lse || !lam || !halt || !argmax || !tokens || !commit_loop || !embed_out)
    return c->fail(ALODLM_EINVAL, "null pointer");
  if (n_rows < 1 || n_rows > c->plan.rows_step) return c->fail(ALODLM_EINVAL, "n_rows outside 1..max_batch*max_block");
  if (group < 1 || group > 64 || n_rows % group) return c->fail(ALODLM_EINVAL, "group must be 1..64 and divide n_rows");
  // the per-sequence state (commit counts, stop flags, active lists) holds max_batch sequences
  if (n_rows / group > g.max_batch) return c->fail(ALODLM_EINVAL, "n_rows / group exceeds max_batch sequences");
  if (boost_tok && !boost_val) return c->fail(ALODLM_EINVAL, "boost_tok without boost_val");
  if (!finite_f(tau_ent) || !finite_f(tau_halt)) return c->fail(ALODLM_EINVAL, "non-finite threshold");
  return ALODLM_OK;
}

// The readout half of one loop on given rows: every buffer it writes besides the outputs is in `sc`
// (launch_step_init sets every entry that is read before it is written).
int readout_run(alodlm_ctx* c, const ReadoutScratch& sc, const void* rows, int32_t n_rows, int32_t group,
                float tau_ent, float tau_halt, const int32_t* boost_tok, const float* boost_val, float* entropy,
                float* lse, float* lam, float* halt, int32_t* argmax, int32_t* tokens, int8_t* commit_loop,
                float* embed_out) {
  const alodlm_config& g = c->cfg;
  const int B = n_rows / group, L = group;
  hipStream_t st = c->st;
  launch_step_init(nullptr, B, L, g.mask_id, sc.U, halt, tokens, commit_loop, sc.ncommit, sc.stop, sc.seq_loops,
                   sc.act0, sc.src_slot, st);
  launch_build_lists(B, L, B, 1, sc.act0, sc.stop, sc.U, sc.ncommit, sc.act1, sc.src_slot, sc.ro_rows, sc.ro_map,
                     sc.cnt, st);
  launch_exit_gate(dt(c), rows, n_rows, g.d_model, c->w.exit_w, c->w.exit_b, lam, st);
  // LMHead over the given rows (row order = readout order)
  GemmEpi ep;
  ep.part = sc.part;
  ep.n_tiles = lm_tiles(c, n_rows);
  ep.btok = boost_tok;
  ep.bval = boost_val;
  lm_head_gemm(c, rows, n_rows, nullptr, ep);
  launch_softstat_combine(sc.part, n_rows, ep.n_tiles, nullptr, entropy, lse, argmax, nullptr, nullptr, st);
  c->dbg_point("readout of rows", n_rows);
  // one loop of the commit rule (a starts at 0, so a = lambda); per-row records go to the outputs
  launch_commit(B, 1, 1, L, B, tau_ent, tau_halt, sc.act1, sc.U, halt, sc.ro_map, entropy, argmax, nullptr, lam, lse,
                tokens, commit_loop, sc.ncommit, sc.stop, sc.seq_loops, nullptr, nullptr, nullptr, nullptr, nullptr,
                nullptr, nullptr, nullptr, nullptr, st);
  launch_embed_committed(dt(c), commit_loop, tokens, c->w.embed, n_rows, g.d_model, g.vocab, embed_out, st);
  c->dbg_point("commit of rows", n_rows);
  return c->hip_check("readout launch");
}

constexpr size_t kStaticScratchBytes = (size_t)ALODLM_STATIC_SCRATCH_BYTES;
}  // namespace

// Scratch of the allocation-free readout (alodlm_readout_commit_static): one array per device,
// held until the process ends.  Host code never passes the array's name to a kernel (on the host
// it names a host-side stand-in); it uses the device address looked up once per device.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {nullptr};

// Device address of the current device's array, looked up on the first call on that device.
int static_scratch(void** out, std::string* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = std::string("hipGetDevice: ") + (e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    return ALODLM_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return ALODLM_EHIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return ALODLM_OK;
}

// Carves the readout scratch for n_rows rows of `group` out of `base` (nullptr: sizes only);
// returns the bytes used.
size_t carve_readout(char* base, int n_rows, int group, int n_tiles, ReadoutScratch* sc) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  const size_t B = (size_t)(n_rows / group);
  sc->part = (SoftStat*)take(sizeof(SoftStat) * (size_t)n_rows * n_tiles);
  sc->U = (uint8_t*)take((size_t)n_rows);
  sc->ro_map = (int32_t*)take(sizeof(int32_t) * n_rows);
  sc->ro_rows = (int32_t*)take(sizeof(int32_t) * n_rows);
  sc->act0 = (int32_t*)take(sizeof(int32_t) * B);
  sc->act1 = (int32_t*)take(sizeof(int32_t) * B);
  sc->src_slot = (int32_t*)take(sizeof(int32_t) * B);
  sc->ncommit = (int32_t*)take(sizeof(int32_t) * B);
  sc->stop = (uint8_t*)take(B);
  sc->seq_loops = (int8_t*)take(B);
  sc->cnt = (int32_t*)take(sizeof(int32_t) * 8);
  return off;
}
}  // namespace

extern "C" {

int alodlm_readout_commit(alodlm_ctx* c, const void* rows, int32_t n_rows, int32_t group, float tau_ent,
                          float tau_halt, const int32_t* boost_tok, const float* boost_val, float* entropy, float* lse,
                          float* lam, float* halt, int32_t* argmax, int32_t* tokens, int8_t* commit_loop,
                          float* embed_out) {
  if (!c) return ALODLM_EINVAL;
  if (int rc = readout_check(c, rows, n_rows, group, tau_ent, tau_halt, boost_tok, boost_val, entropy, lse, lam, halt,
                             argmax, tokens, commit_loop, embed_out))
    return rc;
  if (int rc0 = ensure_device(c)) return rc0;
  const Plan& p = c->plan;
  ReadoutScratch sc;
  sc.part = c->at<SoftStat>(p.part);
  sc.U = c->at<uint8_t>(p.U);
  sc.ro_map = c->at<int32_t>(p.ro_map);
  sc.ro_rows = c->at<int32_t>(p.ro_rows);
  sc.act0 = c->at<int32_t>(p.act_seq0);
  sc.act1 = c->at<int32_t>(p.act_seq1);
  sc.src_slot = c->at<int32_t>(p.src_slot);
  sc.ncommit = c->at<int32_t>(p.ncommit);
  sc.stop = c->at<uint8_t>(p.stop);
  sc.seq_loops = c->at<int8_t>(p.seq_loops);
  sc.cnt = c->at<int32_t>(p.cnt);
  return readout_run(c, sc, rows, n_rows, group, tau_ent, tau_halt, boost_tok, boost_val, entropy, lse, lam, halt,
                     argmax, tokens, commit_loop, embed_out);
}

int alodlm_readout_commit_static(alodlm_ctx* c, const void* rows, int32_t n_rows, int32_t group, float tau_ent,
                                 float tau_halt, const int32_t* boost_tok, const float* boost_val, float* entropy,
                                 float* lse, float* lam, float* halt, int32_t* argmax, int32_t* tokens,
                                 int8_t* commit_loop, float* embed_out) {
  if (!c) return ALODLM_EINVAL;
  if (int rc = readout_check(c, rows, n_rows, group, tau_ent, tau_halt, boost_tok, boost_val, entropy, lse, lam, halt,
                             argmax, tokens, commit_loop, embed_out))
    return rc;
  ReadoutScratch sc;
  const size_t need = carve_readout(nullptr, n_rows, group, lm_tiles(c, n_rows), &sc);
  if (need > kStaticScratchBytes)
    return c->fail(ALODLM_EINVAL, "readout needs " + std::to_string(need) + " bytes of scratch, the fixed array holds " +
                                      std::to_string(kStaticScratchBytes));
  void* base = nullptr;
  std::string err;
  if (int rc = static_scratch(&base, &err)) return c->fail(rc, err);
  carve_readout((char*)base, n_rows, group, lm_tiles(c, n_rows), &sc);
  return readout_run(c, sc, rows, n_rows, group, tau_ent, tau_halt, boost_tok, boost_val, entropy, lse, lam, halt,
                     argmax, tokens, commit_loop, embed_out);
}

int alodlm_diag_timing_enable(alodlm_ctx* c, int32_t enable) {
  if (!c) return ALODLM_EINVAL;
  c->timing = enable != 0;
  c->ev_used = 0;
  for (int k = 0; k < ALODLM_K_CLASSES; ++k) {
    c->t_ms[k] = 0.0;
    c->t_n[k] = 0;
  }
  return ALODLM_OK;
}

int alodlm_diag_timing_read(const alodlm_ctx* c, int32_t kernel_class, double* ms, int64_t* launches) {
  if (!c || kernel_class < 0 || kernel_class >= ALODLM_K_CLASSES) return ALODLM_EINVAL;
  if (ms) *ms = c->t_ms[kernel_class];
  if (launches) *launches = c->t_n[kernel_class];
  return ALODLM_OK;
}

int alodlm_diag_read_kv(const alodlm_ctx* c, int32_t slot, int32_t b, int32_t j0, int32_t n, void* dst_k,
                        void* dst_v) {
  if (!c || !dst_k || !dst_v) return ALODLM_EINVAL;
  const alodlm_config& g = c->cfg;
  if (slot < 0 || slot >= c->plan.n_slots || b < 0 || b >= g.max_batch || j0 < 0 || n < 0 ||
      j0 + n > g.max_prefix)
    return ALODLM_EINVAL;
  if (ensure_device(const_cast<alodlm_ctx*>(c))) return ALODLM_EHIP;
  const size_t es = kv_esize(g), hd = g.head_dim, Pp = (size_t)c->plan.Pp;
  const char* kbase = c->ws + c->plan.kcache + es * (size_t)c->plan.slot_elems * slot;
  for (int h = 0; h < g.n_kv_heads; ++h) {
    const char* src = kbase + es * (((size_t)b * g.n_kv_heads + h) * Pp + j0) * hd;
    char* dst = (char*)dst_k + es * (size_t)h * n * hd;
    if (hipMemcpyAsync(dst, src, es * n * hd, hipMemcpyDeviceToDevice, c->st) != hipSuccess) return ALODLM_EHIP;
  }
  const char* vbase = c->ws + c->plan.vcache + es * (size_t)c->plan.slot_elems * slot;
  launch_read_v_rows(g.kv_dtype == ALODLM_KV_FP8 ? DT_FP8 : (g.dtype == ALODLM_DTYPE_BF16 ? DT_BF16 : DT_FP32), vbase, b,
                     g.n_kv_heads, (int)Pp, (int)hd, j0,
                     n, dst_v, c->st);
  return hipGetLastError() == hipSuccess ? ALODLM_OK : ALODLM_EHIP;
}

int64_t alodlm_diag_buffer_offset(const alodlm_ctx* c, const char* name) {
  if (!c || !name) return -1;
  const Plan& p = c->plan;
  const struct {
    const char* n;
    size_t off;
  } tab[] = {{"h", p.h}, {"xn", p.xn}, {"attn", p.attn}, {"q", p.q}, {"qkv", p.qkv}, {"act", p.act}, {"r", p.r}};
  for (const auto& t : tab)
    if (!strcmp(t.n, name)) return (int64_t)t.off;
  return -1;
}

int alodlm_last_step_stats(const alodlm_ctx* c, int64_t* layer_calls, int32_t* loops_run) {
  if (!c) return ALODLM_EINVAL;
  if (layer_calls) *layer_calls = c->layer_calls;
  if (loops_run) *loops_run = c->loops_run;
  return ALODLM_OK;
}

const char* alodlm_last_error(const alodlm_ctx* c) { return c ? c->err.c_str() : g_create_error.c_str(); }

void alodlm_destroy(alodlm_ctx* c) { delete c; }

}  // extern "C"
