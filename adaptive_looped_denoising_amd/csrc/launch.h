// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alodlm {

enum { DT_BF16 = 0, DT_FP32 = 1, DT_FP8 = 2 };  // DT_FP8: K/V storage only (OCP E4M3)
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SOFTSTAT = 2, EPI_SWIGLU = 3 };

struct SoftStat;
struct GStat;

// Sampling parameters of a readout: Philox key and counter words 2 and 3; row_key[m] is counter
// word 1 of readout row m (64 * sequence + block row).  Word 0 is the column divided by 4 and
// column mod 4 picks the output word.
struct SampleParams {
  const int32_t* row_key = nullptr;
  GStat* part = nullptr;  // [rows][column tiles] partial draws
  uint32_t k0 = 0, k1 = 0, c2 = 0, c3 = 0;
};

// GEMM epilogue operands.  STORE: C = acc.  RESID: C = R + acc (fp32, R may alias C).
// SOFTSTAT: per (row, column tile) softmax statistics of acc + boost into part[row][tile].
// SWIGLU: act[row][j] = silu(gate_j) * up_j (act in the activation dtype).
struct GemmEpi {
  float* C = nullptr;
  const float* R = nullptr;
  int ldc = 0;
  SoftStat* part = nullptr;
  int n_tiles = 0;
  const int32_t* btok = nullptr;
  const float* bval = nullptr;
  void* act = nullptr;
  int ld_act = 0;
  SampleParams smp;  // SOFTSTAT with smp.part: also the Gumbel-max draw of each row and tile
  int col0 = 0;      // SOFTSTAT over a column range: vocabulary id of the launch's column 0
};

// Attention operands.  Query rows r = t * rows_per_seq + i of sequence slot t (cache sequence
// seq_map[t], or t).  Keys: n_cache prefix keys at ck/cv + b*c_sSeq + h*c_sHead + j*c_sPos
// (+ (min(loop, avail[b*av_stride + j]) - 1) * c_plane for Core layers), then the rows' own
// keys at sk/sv + (t + s_seq0)*s_sSeq + h*s_sHead + jj*s_sPos (jj <= i when causal).
// Attention operands.  Keys are the prefix keys j < n_cache (cache slot, already the right depth
// plane) followed by the rows' own keys (n_self of them).  K rows are hd-contiguous:
// k(j) = base + seq * kSeq + kvh * kHead + j * kPos.  V is stored transposed, positions
// contiguous: v(j, e) = base + seq * vSeq + kvh * vHead + e * vRow + j, with vRow a multiple of
// 64 (whole 64-key tiles stay inside a row).
struct AttnParams {
  const void* q = nullptr;  // [n_rows][Hq][hd]
  void* out = nullptr;      // [n_rows][Hq*hd]
  int n_rows = 0, rows_per_seq = 1, Hq = 1, Hkv = 1, hd = 0;
  float scale = 1.f;
  const void* ck = nullptr;
  const void* cv = nullptr;
  int64_t c_kSeq = 0, c_kHead = 0, c_kPos = 0, c_vSeq = 0, c_vHead = 0, c_vRow = 0;
  int n_cache = 0;
  const int32_t* seq_map = nullptr;  // sequence slot t -> cache sequence (null: identity)
  const void* sk = nullptr;
  const void* sv = nullptr;
  int64_t s_kSeq = 0, s_kHead = 0, s_kPos = 0, s_vSeq = 0, s_vHead = 0, s_vRow = 0;
  // causal: query row i sees own key jj iff jj <= i + causal_off (rows appended after
  // causal_off own keys that are already in place)
  int n_self = 0, causal = 0, s_seq0 = 0, causal_off = 0;
  int kv8 = 0;  // keys and values (cache and own) stored in FP8 E4M3 (matrix-core path, hd 64 / 128)
  // fast path scratch: split-KV partials
  float* part = nullptr;
  int n_split = 1;
};

void launch_embed_rows(int dtype, const int32_t* ids, int n_rows, const void* E, int d, int V, float* out,
                       hipStream_t st);
// x rows are x[src] (+ sum of `splits` deferred split-K partials part[s][r][:] when splits > 1,
// written back to x_out[r]).  Output row r at out + r * out_ld (0: d).
void launch_rmsnorm(int dtype, const float* x, int n_rows, int d, const int32_t* rows, const int32_t* n_dev,
                    const void* g, float eps, void* out, const void* exit_w, float exit_b, float* lam,
                    hipStream_t st, const float* part = nullptr, int splits = 1, float* x_out = nullptr,
                    int out_ld = 0);
void launch_exit_gate(int dtype, const void* rows, int n_rows, int d, const void* w, float b, float* lam,
                      hipStream_t st);
// qkv rows come from `qkv`, or are the sum of `splits` deferred split-K partials [s][row][:] of
// the projection when splits > 1 (qkv then points at the partials).
// K rows go to k_out + seq * kSeq + kvh * kHead + pos * kPos (hd-contiguous), V transposed to
// v_out + seq * vSeq + kvh * vHead + e * vRow + pos, seq = seq0 + row / rows_per_seq.
void launch_qk_norm_rope(int dtype, const float* qkv, int n_rows, int rows_per_seq, int pos0, int Hq, int Hkv,
                         int hd, const void* qn, const void* kn, float eps, const float* cosT, const float* sinT,
                         void* q_out, void* k_out, void* v_out, int64_t kSeq, int64_t kHead, int64_t kPos,
                         int64_t vSeq, int64_t vHead, int64_t vRow, int seq0, hipStream_t st, int splits = 1, int kv_type = -1);
void launch_swiglu(int dtype, const float* gu, int n_rows, int F, void* act, hipStream_t st);
// gpart (optional): partial Gumbel-max draws merged into stok (the sampled token of each row).
void launch_softstat_combine(const SoftStat* part, int n_rows, int n_tiles, const int32_t* n_dev, float* H,
                             float* lse, int32_t* tok, const GStat* gpart, int32_t* stok, hipStream_t st);
void launch_step_init(const int32_t* block_ids, int B, int L, int mask_id, uint8_t* U, float* a, int32_t* tokens,
                      int8_t* cl, int32_t* ncommit, uint8_t* stop, int8_t* loops, int32_t* act, int32_t* src_slot,
                      hipStream_t st);
void launch_build_lists(int nb, int L, int B, int keep_all, const int32_t* act_cur, const uint8_t* stop,
                        const uint8_t* U, const int32_t* ncommit, int32_t* act_next, int32_t* src_slot, int32_t* ro_rows,
                        int32_t* ro_map, int32_t* cnt, hipStream_t st);
// stok (optional): sampled token per readout row, committed instead of the argmax tok.
void launch_commit(int nb, int s, int k_loops, int L, int B, float tau_ent, float tau_halt, const int32_t* act,
                   uint8_t* U, float* a, const int32_t* ro_map, const float* H, const int32_t* tok,
                   const int32_t* stok, const float* lam, const float* lse, int32_t* tokens, int8_t* cl,
                   int32_t* ncommit, uint8_t* stop, int8_t* loops, const int8_t* tf_cl, const int32_t* tf_tok,
                   const int8_t* tf_stop, float* dbg_H, float* dbg_lam, float* dbg_a, float* dbg_lse,
                   int32_t* dbg_tok, int32_t* dbg_stok, hipStream_t st);
void launch_reset_compact(int dtype, int nb_upper, const int32_t* cnt, int L, int d, int V, const int32_t* act,
                          const int32_t* src, const uint8_t* U, const int32_t* tokens, const float* h_old,
                          const void* E, float* h_new, hipStream_t st);
void launch_dump_hidden(int nb, int L, int d, int B, int s, const int32_t* act, const float* h, float* out,
                        hipStream_t st);
// Per readout row k (sequence b, block row i): its boost (when boost_tok is given) and its
// sampling row key 64 * b + i (when rkey is given).
void launch_gather_rows(const int32_t* ro_rows, const int32_t* n_dev, const int32_t* act, int n_upper, int L,
                        const int32_t* boost_tok, const float* boost_val, int32_t* btok, float* bval, int32_t* rkey,
                        hipStream_t st);
// Outer loop over a block: init copies the block ids, clears the commit records and counts the
// masked positions into cnt[0]; merge records step t's commits and takes its output ids.
void launch_block_init(const int32_t* block_ids, int n, int mask_id, int32_t* ids, int16_t* commit_step,
                       int8_t* commit_loop, int32_t* cnt, hipStream_t st);
void launch_block_merge(int n, int t, const int32_t* step_tok, const int8_t* step_cl, int32_t* ids,
                        int16_t* commit_step, int8_t* commit_loop, hipStream_t st);
void launch_embed_committed(int dtype, const int8_t* cl, const int32_t* tokens, const void* E, int n, int d, int V,
                            float* out, hipStream_t st);

bool gemm_mfma_supported(int K, int lda, int ldb);
// Column-tile width the matrix-core dispatcher uses for a SOFTSTAT (LM-head) GEMM of M rows:
// the softmax statistics are kept per column tile.
// Column ranges of an M-row LM-head readout over N columns on the matrix cores: columns
// [0, cols0) on tile0 (tiles0 column tiles), then, if tile1 >= 0, columns [cols0, N) on tile1;
// n_tiles = the per-row partial statistics of both (column-tile order).
struct SoftstatPlan {
  int tile0, cols0, tiles0, tile1, n_tiles;
};
void gemm_mfma_softstat_plan(int M, int N, int force_tile, SoftstatPlan* plan);
// Returns the number of split-K partials left unreduced in `part` ([splits][M][N] fp32, plain
// A.B^T sums) when defer_reduce is set and the GEMM was split (STORE / RESID only), else 1 (the
// epilogue has been applied).
int launch_gemm_mfma(int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                     const int32_t* m_dev, const GemmEpi& ep, int F, float* part, size_t part_floats,
                     int force_splits, hipStream_t st, int force_tile = -1, bool defer_reduce = false);
void launch_gemm_generic(int dtype, int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                         const int32_t* m_dev, const GemmEpi& ep, hipStream_t st);
void launch_attn_generic(int dtype, const AttnParams& p, hipStream_t st);
bool attn_mfma_supported(int hd);
void launch_attn_mfma(const AttnParams& p, int max_splits, hipStream_t st, int force_splits = 0, int force_qw = 0,
                      int force_ns = 0, int force_nw = 0, int force_kh = 0);

// Cache slot fill with the counter-based synthetic values: logical element (b, kvh, j, e) is
// generator index ((b * Hkv + kvh) * P + j) * hd + e; stored K-layout ([b][kvh][P_pitch][hd]) or,
// with transposed, V-layout ([b][kvh][hd][P_pitch]).
void launch_fill_kv_synth(int dtype, void* slot_base, int B, int Hkv, int P, int P_pitch, int hd, uint32_t seed,
                          uint32_t tensor, float scale, bool transposed, hipStream_t st);
// Available-depth table [B][pitch]: positions j0 .. j0+n-1 of each sequence from src [B][n], or
// the value v when src is null, clipped to cap (the Core depths the cache keeps).
void launch_set_avail(uint8_t* dst, int pitch, int j0, int B, int n, const uint8_t* src, uint8_t v, uint8_t cap,
                      hipStream_t st);
// Depth planes of one Core layer's cache (plane p = depth p + 1, plane_elems apart): for every
// position j with avail[b][j] = a_j, plane p takes the values of plane max(1, min(p + 1, a_j)) - 1,
// so that reading plane s - 1 at loop s gives every key at depth min(s, a_j).
void launch_materialize_depth(int dtype, void* k_plane0, void* v_plane0, int64_t plane_elems, int k_max, int B,
                              int Hkv, int j0, int n_pos, int P_pitch, int hd, const uint8_t* avail, int av_pitch,
                              hipStream_t st);
// V rows j0 .. j0+n-1 of a transposed cache slot, every kv head, to dst [Hkv][n][hd].
void launch_read_v_rows(int dtype, const void* slot_base, int b, int Hkv, int P_pitch, int hd, int j0, int n,
                        void* dst, hipStream_t st);

}  // namespace alodlm
