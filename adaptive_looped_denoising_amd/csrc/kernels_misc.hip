// Row-wise kernels of the looped denoising step: embedding gather, RMSNorm (+ the
// ExitGate head), per-head q/k RMSNorm + RoPE (+ prefix-cache write), SwiGLU,
// the vocabulary-partial combine, the commit / halting / forced-progress rule,
// the active-list compaction and the Eq. 3 state reset.
#include "common.h"
#include "launch.h"

namespace alodlm {

// ---------------------------------------------------------------------------------------------
// h[r] = Emb[ids[r]]  (fp32 residual rows)
template <typename T>
__global__ __launch_bounds__(256) void k_embed_rows(const int32_t* __restrict__ ids, const T* __restrict__ E,
                                                    int d, int V, float* __restrict__ out) {
  const int r = blockIdx.x;
  const T* src = E + (size_t)min(max(ids[r], 0), V - 1) * d;
  float* dst = out + (size_t)r * d;
  for (int e = threadIdx.x; e < d; e += blockDim.x) dst[e] = to_f(src[e]);
}

// ---------------------------------------------------------------------------------------------
// out[r] = x[src(r)] / sqrt(mean(x^2) + eps) * g ; optional ExitGate lambda = sigmoid(w . out + b)
// computed on the fp32 normalised row.  Rows >= *n_dev (when given) are skipped.  The row stays
// in registers between the two reductions (16-byte loads, d <= 256 * 4 * RMS_VEC).
constexpr int RMS_VEC = 8;

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  uint2 w;
  w.x = (uint32_t)from_f<bf16_t>(a) | ((uint32_t)from_f<bf16_t>(b) << 16);
  w.y = (uint32_t)from_f<bf16_t>(c) | ((uint32_t)from_f<bf16_t>(d) << 16);
  *(uint2*)p = w;
}
template <typename T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *(const float4*)p;
}
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
  const uint2 w = *(const uint2*)p;
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u));
}

// SPLITS (compile time, 0 = runtime `splits`): the number of deferred split-K partials to add, so
// that every partial load of the row can be in flight at once.
template <typename TG, typename TO, int SPLITS>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, int d,
                                                 const int32_t* __restrict__ rows,
                                                 const int32_t* __restrict__ n_dev, const TG* __restrict__ g,
                                                 float eps, TO* __restrict__ out, const TG* __restrict__ exit_w,
                                                 float exit_b, float* __restrict__ lam,
                                                 const float* __restrict__ part, int splits_rt, int n_rows_part,
                                                 float* __restrict__ x_out, int out_ld) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  if (n_dev && r >= *n_dev) return;
  const int splits = SPLITS > 0 ? SPLITS : splits_rt;
  const int src = rows ? rows[r] : r;
  const float* xr = x + (size_t)src * d;
  float4 v[RMS_VEC];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RMS_VEC; ++i) {
    const int e = (i * 256 + threadIdx.x) * 4;
    v[i] = e < d ? *(const float4*)(xr + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (splits > 1) {  // residual + fixed-order sum of the producing GEMM's split-K partials
#pragma unroll
    for (int i = 0; i < RMS_VEC; ++i) {
      const int e = (i * 256 + threadIdx.x) * 4;
      if (e >= d) continue;
      float4 pp[SPLITS > 0 ? SPLITS : 1];
      float4 acc;
      if (SPLITS > 0) {
#pragma unroll
        for (int sp = 0; sp < (SPLITS > 0 ? SPLITS : 1); ++sp)
          pp[sp] = *(const float4*)(part + ((size_t)sp * n_rows_part + src) * d + e);
        acc = pp[0];
#pragma unroll
        for (int sp = 1; sp < (SPLITS > 0 ? SPLITS : 1); ++sp) {
          acc.x += pp[sp].x;
          acc.y += pp[sp].y;
          acc.z += pp[sp].z;
          acc.w += pp[sp].w;
        }
      } else {
        acc = *(const float4*)(part + (size_t)src * d + e);
        for (int sp = 1; sp < splits; ++sp) {
          const float4 q = *(const float4*)(part + ((size_t)sp * n_rows_part + src) * d + e);
          acc.x += q.x;
          acc.y += q.y;
          acc.z += q.z;
          acc.w += q.w;
        }
      }
      v[i].x += acc.x;
      v[i].y += acc.y;
      v[i].z += acc.z;
      v[i].w += acc.w;
      *(float4*)(x_out + (size_t)src * d + e) = v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < RMS_VEC; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  ss = block_sum<256>(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  float dot = 0.f;
  TO* o = out + (size_t)r * out_ld;
#pragma unroll
  for (int i = 0; i < RMS_VEC; ++i) {
    const int e = (i * 256 + threadIdx.x) * 4;
    if (e < d) {
      const float4 gg = load4<TG>(g + e);
      const float a = v[i].x * inv * gg.x, b = v[i].y * inv * gg.y, c = v[i].z * inv * gg.z, dd = v[i].w * inv * gg.w;
      store4<TO>(o + e, a, b, c, dd);
      if (exit_w) {
        const float4 ww = load4<TG>(exit_w + e);
        dot += a * ww.x + b * ww.y + c * ww.z + dd * ww.w;
      }
    }
  }
  if (exit_w) {
    dot = block_sum<256>(dot, red);
    if (threadIdx.x == 0) lam[r] = 1.0f / (1.0f + expf(-(dot + exit_b)));
  }
}

// ExitGate on given readout rows: lambda = sigmoid(w . r + b).
template <typename T>
__global__ __launch_bounds__(256) void k_exit_gate(const T* __restrict__ rows, int d, const T* __restrict__ w,
                                                   float b, float* __restrict__ lam) {
  __shared__ float red[4];
  const T* rr = rows + (size_t)blockIdx.x * d;
  float dot = 0.f;
  for (int e = threadIdx.x; e < d; e += 256) dot += to_f(rr[e]) * to_f(w[e]);
  dot = block_sum<256>(dot, red);
  if (threadIdx.x == 0) lam[blockIdx.x] = 1.0f / (1.0f + expf(-(dot + b)));
}

// ---------------------------------------------------------------------------------------------
// Per-head RMSNorm of q and k, rotary embedding (rotate-half pairs (p, p + hd/2)), and the
// layout change of q/k/v.  Blocks 0 .. qk_blocks-1: each wave takes QK_PER_WAVE consecutive
// (row, q or k head) items (4 for prefill-sized row counts, whose waves would otherwise each wait
// on one round trip, 1 for a step's few rows); lane p owns the pair (p, p + hd/2); K element (row r, kv head h, e) goes to
// k_out + (seq0 + r / n)*kSeq + h*kHead + (r % n)*kPos + e.  The remaining blocks transpose the
// value heads: one block per (sequence, kv head, chunk of up to 64 positions, 32 of the hd
// elements) stages the chunk in LDS and writes each V^T row v_out + seq*vSeq + h*vHead +
// e*vRow + position as one contiguous run (a wave per (row, head) would scatter 2-byte writes
// vRow apart).
// SPLITS (compile time, 0 = runtime `splits`): split-K partials of the projection to add.
// TKV: storage type of the keys and values (the activation type, or FP8 E4M3).
template <typename TW, typename TA, typename TKV, int SPLITS, int QK_PER_WAVE>
__global__ __launch_bounds__(256) void k_qk_norm_rope(const float* __restrict__ qkv, int n_rows, int rows_per_seq,
                                                      int pos0, int Hq, int Hkv, int hd,
                                                      const TW* __restrict__ qn, const TW* __restrict__ kn,
                                                      float eps, const float* __restrict__ cosT,
                                                      const float* __restrict__ sinT, TA* __restrict__ q_out,
                                                      TKV* __restrict__ k_out, TKV* __restrict__ v_out,
                                                      int64_t kSeq, int64_t kHead, int64_t kPos, int64_t vSeq,
                                                      int64_t vHead, int64_t vRow, int seq0, int splits_rt,
                                                      int qk_blocks) {
  const int splits = SPLITS > 0 ? SPLITS : splits_rt;
  const int NH = Hq + 2 * Hkv;
  const size_t pstride = (size_t)n_rows * NH * hd;  // split-K partial stride
  // element e of head hh of row r: the projection, or the fixed-order sum of its split-K partials
  auto head_val = [&](int r, int hh, int e) {
    const float* src = qkv + (size_t)r * NH * hd + (size_t)hh * hd;
    float acc = src[e];
    if (SPLITS > 0) {
#pragma unroll
      for (int sp = 1; sp < SPLITS; ++sp) acc += src[sp * pstride + e];
    } else {
      for (int sp = 1; sp < splits; ++sp) acc += src[sp * pstride + e];
    }
    return acc;
  };
  if ((int)blockIdx.x >= qk_blocks) {  // value heads, transposed through LDS
    __shared__ float tile[32][65];
    const int chunks = (rows_per_seq + 63) / 64, slices = hd / 32;
    int vb = blockIdx.x - qk_blocks;
    const int sl = vb % slices;
    vb /= slices;
    const int ch = vb % chunks, h = (vb / chunks) % Hkv, sq = vb / (chunks * Hkv);
    const int j0 = ch * 64, n = min(64, rows_per_seq - j0);
    const int r0 = sq * rows_per_seq + j0, e0 = sl * 32;
    for (int i = threadIdx.x; i < n * 32; i += 256) {
      const int j = i >> 5, e = i & 31;
      tile[e][j] = head_val(r0 + j, Hq + Hkv + h, e0 + e);
    }
    __syncthreads();
    TKV* dst = v_out + (size_t)(seq0 + sq) * vSeq + (size_t)h * vHead + (size_t)e0 * vRow + j0;
    for (int i = threadIdx.x; i < n * 32; i += 256) {
      const int e = i / n, j = i % n;
      dst[(size_t)e * vRow + j] = from_f<TKV>(tile[e][j]);
    }
    return;
  }
  // q/k heads: each wave takes QK_PER_WAVE consecutive (row, head) items and issues the loads of
  // all of them before using any (one item per wave leaves each wave waiting on one round trip)
  const int NQK = Hq + Hkv;
  const int lane = threadIdx.x & 63;
  const int item0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * QK_PER_WAVE;
  const int n_items = n_rows * NQK;
  if (item0 >= n_items) return;
  const int half = hd >> 1;
  float x1[QK_PER_WAVE][2], x2[QK_PER_WAVE][2];
#pragma unroll
  for (int k = 0; k < QK_PER_WAVE; ++k) {
    const int it = min(item0 + k, n_items - 1);
    const int r = it / NQK, hh = it % NQK;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = lane + 64 * t;
      x1[k][t] = x2[k][t] = 0.f;
      if (p < half) {
        x1[k][t] = head_val(r, hh, p);
        x2[k][t] = head_val(r, hh, p + half);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < QK_PER_WAVE; ++k) {
    if (item0 + k >= n_items) break;
    const int r = (item0 + k) / NQK, hh = (item0 + k) % NQK;
    const int jpos = r % rows_per_seq;
    const int pos = pos0 + jpos;
    const size_t seq = (size_t)(seq0 + r / rows_per_seq);
    const size_t kv_off = seq * kSeq + (size_t)jpos * kPos;
    const bool is_q = hh < Hq;
    const TW* g = is_q ? qn : kn;
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) ss += x1[k][t] * x1[k][t] + x2[k][t] * x2[k][t];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
    TA* dq = q_out + ((size_t)r * Hq + hh) * hd;
    TKV* dk = k_out + kv_off + (size_t)(hh - Hq) * kHead;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = lane + 64 * t;
      if (p < half) {
        const float a = x1[k][t] * inv * to_f(g[p]);
        const float b = x2[k][t] * inv * to_f(g[p + half]);
        const float c = cosT[(size_t)pos * half + p], s = sinT[(size_t)pos * half + p];
        const float lo = a * c - b * s, hi = b * c + a * s;
        if (is_q) {
          dq[p] = from_f<TA>(lo);
          dq[p + half] = from_f<TA>(hi);
        } else {
          dk[p] = from_f<TKV>(lo);
          dk[p + half] = from_f<TKV>(hi);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// act[r][j] = silu(gu[r][j]) * gu[r][F + j]
template <typename TA>
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ gu, int n_rows, int F,
                                                TA* __restrict__ act) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)n_rows * F) return;
  const size_t r = i / F, j = i % F;
  const float g = gu[r * 2 * F + j], u = gu[r * 2 * F + F + j];
  act[i] = from_f<TA>(g / (1.0f + expf(-g)) * u);
}

// ---------------------------------------------------------------------------------------------
// Merge the per-tile softmax statistics of each readout row in a fixed order:
// entropy H = ln S - T/S, lse = m + ln S, token = argmax.
// With gpart, also the Gumbel-max draw: the largest z + g over the tiles (lowest column on ties).
__global__ __launch_bounds__(64) void k_softstat_combine(const SoftStat* __restrict__ part, int n_tiles,
                                                         const int32_t* __restrict__ n_dev,
                                                         float* __restrict__ H, float* __restrict__ lse,
                                                         int32_t* __restrict__ tok, const GStat* __restrict__ gpart,
                                                         int32_t* __restrict__ stok) {
  const int r = blockIdx.x;
  if (n_dev && r >= *n_dev) return;
  const SoftStat* p = part + (size_t)r * n_tiles;
  SoftStat s = softstat_empty();
  for (int t = threadIdx.x; t < n_tiles; t += 64) s = softstat_merge(s, p[t]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s = softstat_merge(s, softstat_shfl_xor(s, o));
  if (threadIdx.x == 0) {
    const float lS = logf(s.S);
    H[r] = lS - s.T / s.S;
    lse[r] = s.m + lS;
    tok[r] = s.idx;
  }
  if (gpart) {
    const GStat* q = gpart + (size_t)r * n_tiles;
    float gg = -INFINITY;
    int gi = 0x7FFFFFFF;
    for (int t = threadIdx.x; t < n_tiles; t += 64) gstat_take(gg, gi, q[t].g, q[t].idx);
    gstat_reduce_xor<32>(gg, gi);
    if (threadIdx.x == 0) stok[r] = gi;
  }
}

// ---------------------------------------------------------------------------------------------
// Step state.  Per (sequence b, row i) with stride L: U (1 = unresolved), a (cumulative halt),
// ro_map (readout row index), tokens, commit_loop.  Per sequence: ncommit, stop, loops.
__global__ void k_step_init(const int32_t* __restrict__ block_ids, int n, int mask_id,
                            uint8_t* __restrict__ U, float* __restrict__ a, int32_t* __restrict__ tokens,
                            int8_t* __restrict__ cl, int B, int32_t* __restrict__ ncommit,
                            uint8_t* __restrict__ stop, int8_t* __restrict__ loops, int32_t* __restrict__ act,
                            int32_t* __restrict__ src_slot) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const int id = block_ids ? block_ids[i] : mask_id;
    U[i] = id == mask_id;
    a[i] = 0.f;
    tokens[i] = id;
    cl[i] = 0;
  }
  if (i < B) {
    ncommit[i] = 0;
    stop[i] = 0;
    loops[i] = 0;
    act[i] = i;
    src_slot[i] = i;
  }
}

// Builds the next loop's lists from the current one: surviving sequences keep their order
// (new slot t2 <- old slot t), and the readout rows are their unresolved rows in (slot, row)
// order.  One block; nb <= 1024 sequences.  Also totals the commits of the whole batch.
// cnt[0] = sequences still looping, cnt[1] = readout rows, cnt[2] = committed tokens.
// keep_all (the lists of loop 1, whose launches are sized for the whole batch before any count
// is read back): every sequence keeps its slot, also one with nothing masked, which the commit
// kernel then stops at loop 1 with 0 loops.
__global__ __launch_bounds__(1024) void k_build_lists(int nb, int L, int B, int keep_all,
                                                       const int32_t* __restrict__ act_cur,
                                                       const uint8_t* __restrict__ stop,
                                                       const uint8_t* __restrict__ U,
                                                       const int32_t* __restrict__ ncommit,
                                                       int32_t* __restrict__ act_next,
                                                       int32_t* __restrict__ src_slot,
                                                       int32_t* __restrict__ ro_rows,
                                                       int32_t* __restrict__ ro_map, int32_t* __restrict__ cnt) {
  __shared__ int s_alive[1024];
  __shared__ int s_rows[1024];
  __shared__ int s_commit[1024];
  const int t = threadIdx.x;
  int alive = 0, nrows = 0, b = -1;
  if (t < nb) {
    b = act_cur[t];
    if (!stop[b])
      for (int i = 0; i < L; ++i) nrows += U[b * L + i];
    alive = keep_all || nrows > 0;  // a sequence with nothing unresolved runs no further loop
  }
  int nc = 0;
  for (int bb = t; bb < B; bb += 1024) nc += ncommit[bb];
  s_alive[t] = alive;
  s_rows[t] = nrows;
  s_commit[t] = nc;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scans (Hillis-Steele)
    int va = 0, vr = 0, vc = 0;
    if (t >= o) {
      va = s_alive[t - o];
      vr = s_rows[t - o];
      vc = s_commit[t - o];
    }
    __syncthreads();
    s_alive[t] += va;
    s_rows[t] += vr;
    s_commit[t] += vc;
    __syncthreads();
  }
  if (alive) {
    const int t2 = s_alive[t] - 1;
    int off = s_rows[t] - nrows;
    act_next[t2] = b;
    src_slot[t2] = t;
    for (int i = 0; i < L; ++i) {
      if (U[b * L + i]) {
        ro_rows[off] = t2 * L + i;
        ro_map[b * L + i] = off;
        ++off;
      }
    }
  }
  if (t == 1023) {
    cnt[0] = s_alive[1023];
    cnt[1] = s_rows[1023];
    cnt[2] = s_commit[1023];
  }
}

// The commit rule of one loop, one wave per looping sequence (lane i = block row i, L <= 64):
// cumulative halt a <- a + (1 - a) lambda on rows unresolved at loop start; commit iff
// H <= tau_ent (or the teacher's decision); stop iff no row is left unresolved, the mean a of
// the unresolved rows is >= tau_halt, or s == k_loops (or the teacher's stop loop); a sequence
// that stops without having committed anything in this step commits its unresolved row of
// lowest entropy (lowest row on ties), recorded as -s.  A sequence whose block has no masked
// row denoises nothing: it stops at once and reports 0 loops.
__global__ __launch_bounds__(64) void k_commit(int s, int k_loops, int L, int B, float tau_ent, float tau_halt,
                                               const int32_t* __restrict__ act, uint8_t* __restrict__ U,
                                               float* __restrict__ a, const int32_t* __restrict__ ro_map,
                                               const float* __restrict__ H, const int32_t* __restrict__ tok,
                                               const int32_t* __restrict__ stok,
                                               const float* __restrict__ lam, const float* __restrict__ lse,
                                               int32_t* __restrict__ tokens, int8_t* __restrict__ cl,
                                               int32_t* __restrict__ ncommit, uint8_t* __restrict__ stop,
                                               int8_t* __restrict__ loops, const int8_t* __restrict__ tf_cl,
                                               const int32_t* __restrict__ tf_tok,
                                               const int8_t* __restrict__ tf_stop, float* __restrict__ dbg_H,
                                               float* __restrict__ dbg_lam, float* __restrict__ dbg_a,
                                               float* __restrict__ dbg_lse, int32_t* __restrict__ dbg_tok,
                                               int32_t* __restrict__ dbg_stok) {
  const int b = act[blockIdx.x];
  const int i = threadIdx.x;
  const bool in = i < L;
  const int idx = b * L + i;
  const bool u = in && U[idx];
  float h = NAN, lm = NAN, ls = NAN;
  int tk = -1, sk = -1;
  float av = in ? a[idx] : 0.f;
  if (u) {
    const int k = ro_map[idx];
    h = H[k];
    tk = tok[k];
    sk = stok ? stok[k] : tk;
    lm = lam[k];
    ls = lse[k];
    av = av + (1.0f - av) * lm;
    a[idx] = av;
  }
  bool commit;
  int ctok = sk;  // the committed token: the draw in sampling mode, else the argmax
  if (tf_cl) {
    commit = u && tf_cl[idx] == s;
    if (u) ctok = tf_tok[idx];
  } else {
    commit = u && h <= tau_ent;
  }
  if (commit) {
    tokens[idx] = ctok;
    cl[idx] = (int8_t)s;
    U[idx] = 0;
  }
  const unsigned long long cm = __ballot(commit);
  const bool none = __ballot(u) == 0ull;  // nothing unresolved at loop start: a block without [MASK]
  const bool u2 = u && !commit;
  const unsigned long long um = __ballot(u2);
  const int n_u = __popcll(um);
  const float sum_a = wave_sum(u2 ? av : 0.f);
  int nc = ncommit[b] + __popcll(cm);
  bool st;
  if (tf_stop)
    st = none || s == (int)tf_stop[b];
  else
    st = n_u == 0 || (sum_a / (float)n_u) >= tau_halt || s == k_loops;
  if (st && nc == 0 && n_u > 0) {
    int pick;
    if (tf_cl) {
      const unsigned long long fm = __ballot(u2 && tf_cl[idx] == -s);
      pick = fm ? (__ffsll((long long)fm) - 1) : -1;
    } else {
      // argmin of (H, row) over unresolved rows
      float kh = u2 ? h : INFINITY;
      int ki = u2 ? i : 0x7FFFFFFF;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float oh = __shfl_xor(kh, o, 64);
        const int oi = __shfl_xor(ki, o, 64);
        if (oh < kh || (oh == kh && oi < ki)) {
          kh = oh;
          ki = oi;
        }
      }
      pick = ki < 64 ? ki : -1;
    }
    if (pick >= 0) {
      if (i == pick) {
        tokens[idx] = ctok;
        cl[idx] = (int8_t)(-s);
        U[idx] = 0;
      }
      nc = 1;
    }
  }
  if (i == 0) {
    ncommit[b] = nc;
    stop[b] = st;
    if (st) loops[b] = (int8_t)(none ? 0 : s);
  }
  if (in && dbg_H) {
    const size_t o = (size_t)(s - 1) * B * L + idx;
    dbg_H[o] = h;
    dbg_lam[o] = lm;
    dbg_a[o] = u ? av : NAN;
    dbg_lse[o] = ls;
    dbg_tok[o] = u ? tk : -1;
    if (dbg_stok) dbg_stok[o] = u ? sk : -1;
  }
}

// Next loop's state rows (Eq. 3 and compaction): for new slot t2 (sequence b = act[t2], old slot
// src[t2]), row i keeps its Core output if unresolved, else becomes Emb[token].
template <typename T>
__global__ __launch_bounds__(256) void k_reset_compact(const int32_t* __restrict__ cnt, int L, int d, int V,
                                                       const int32_t* __restrict__ act,
                                                       const int32_t* __restrict__ src,
                                                       const uint8_t* __restrict__ U,
                                                       const int32_t* __restrict__ tokens,
                                                       const float* __restrict__ h_old, const T* __restrict__ E,
                                                       float* __restrict__ h_new) {
  const int r2 = blockIdx.x;
  const int t2 = r2 / L, i = r2 % L;
  if (t2 >= cnt[0]) return;
  const int b = act[t2];
  float* dst = h_new + (size_t)r2 * d;
  if (U[b * L + i]) {
    const float* s = h_old + ((size_t)src[t2] * L + i) * d;
    for (int e = threadIdx.x; e < d; e += 256) dst[e] = s[e];
  } else {
    const T* s = E + (size_t)min(max(tokens[b * L + i], 0), V - 1) * d;
    for (int e = threadIdx.x; e < d; e += 256) dst[e] = to_f(s[e]);
  }
}

// hidden[s-1][b][i][:] = h[t*L + i][:] for the looping sequences.
__global__ __launch_bounds__(256) void k_dump_hidden(int nb, int L, int d, int B, int s,
                                                     const int32_t* __restrict__ act,
                                                     const float* __restrict__ h, float* __restrict__ out) {
  const int r = blockIdx.x;
  const int t = r / L, i = r % L;
  if (t >= nb) return;
  const int b = act[t];
  float* dst = out + (((size_t)(s - 1) * B + b) * L + i) * d;
  const float* s_ = h + (size_t)r * d;
  for (int e = threadIdx.x; e < d; e += 256) dst[e] = s_[e];
}

// Readout row k stands for sequence act[r / L], block row r % L with r = ro_rows[k]: gathers its
// boost and writes its sampling row key 64 * sequence + row.
__global__ void k_gather_rows(const int32_t* __restrict__ ro_rows, const int32_t* __restrict__ n_dev,
                              const int32_t* __restrict__ act, int n_upper, int L,
                              const int32_t* __restrict__ boost_tok, const float* __restrict__ boost_val,
                              int32_t* __restrict__ btok, float* __restrict__ bval, int32_t* __restrict__ rkey) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n_upper || k >= *n_dev) return;
  const int r = ro_rows[k];
  const int b = act[r / L], i = r % L;
  const int src = b * L + i;
  if (boost_tok) {
    btok[k] = boost_tok[src];
    bval[k] = boost_val[src];
  }
  if (rkey) rkey[k] = 64 * b + i;
}

// Outer loop over a block.  k_block_init: working ids = block ids, commit records cleared and
// cnt[0] = masked positions (one block, fixed-order sum).
__global__ __launch_bounds__(1024) void k_block_init(const int32_t* __restrict__ block_ids, int n, int mask_id,
                                                     int32_t* __restrict__ ids, int16_t* __restrict__ commit_step,
                                                     int8_t* __restrict__ commit_loop, int32_t* __restrict__ cnt) {
  __shared__ float red[16];
  int m = 0;
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int id = block_ids[i];
    ids[i] = id;
    commit_step[i] = 0;
    commit_loop[i] = 0;
    m += id == mask_id;
  }
  const float s = block_sum<1024>((float)m, red);
  if (threadIdx.x == 0) cnt[0] = (int32_t)s;
}

// After step t of the outer loop: positions the step committed record (t, its commit loop); the
// working ids become the step's output (committed tokens written in, mask_id where unresolved).
__global__ void k_block_merge(int n, int t, const int32_t* __restrict__ step_tok, const int8_t* __restrict__ step_cl,
                              int32_t* __restrict__ ids, int16_t* __restrict__ commit_step,
                              int8_t* __restrict__ commit_loop) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int8_t cl = step_cl[i];
  if (cl != 0) {
    commit_step[i] = (int16_t)t;
    commit_loop[i] = cl;
  }
  ids[i] = step_tok[i];
}

// embed_out[k] = committed(k) ? Emb[tokens[k]] : 0
template <typename T>
__global__ __launch_bounds__(256) void k_embed_committed(const int8_t* __restrict__ cl,
                                                         const int32_t* __restrict__ tokens, const T* __restrict__ E,
                                                         int d, int V, float* __restrict__ out) {
  const int k = blockIdx.x;
  float* dst = out + (size_t)k * d;
  if (cl[k] != 0) {
    const T* s = E + (size_t)min(max(tokens[k], 0), V - 1) * d;
    for (int e = threadIdx.x; e < d; e += 256) dst[e] = to_f(s[e]);
  } else {
    for (int e = threadIdx.x; e < d; e += 256) dst[e] = 0.f;
  }
}

// ---------------------------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------------------------
#define DISPATCH_T(dtype, T, ...)          \
  if ((dtype) == DT_BF16) {                \
    typedef bf16_t T;                      \
    __VA_ARGS__;                           \
  } else {                                 \
    typedef float T;                       \
    __VA_ARGS__;                           \
  }

void launch_embed_rows(int dtype, const int32_t* ids, int n_rows, const void* E, int d, int V, float* out,
                       hipStream_t st) {
  if (n_rows <= 0) return;
  DISPATCH_T(dtype, T, k_embed_rows<T><<<n_rows, 256, 0, st>>>(ids, (const T*)E, d, V, out));
}

void launch_rmsnorm(int dtype, const float* x, int n_rows, int d, const int32_t* rows, const int32_t* n_dev,
                    const void* g, float eps, void* out, const void* exit_w, float exit_b, float* lam,
                    hipStream_t st, const float* part, int splits, float* x_out, int out_ld) {
  if (n_rows <= 0) return;
  if (out_ld <= 0) out_ld = d;
#define RMS_GO(S)                                                                                              \
  DISPATCH_T(dtype, T,                                                                                         \
             k_rmsnorm<T, T, S><<<n_rows, 256, 0, st>>>(x, d, rows, n_dev, (const T*)g, eps, (T*)out,          \
                                                         (const T*)exit_w, exit_b, lam, part, splits, n_rows, x_out, \
                                                         out_ld))
  if (splits <= 1) {
    RMS_GO(1);
  } else if (splits == 2) {
    RMS_GO(2);
  } else if (splits == 4) {
    RMS_GO(4);
  } else if (splits == 8) {
    RMS_GO(8);
  } else {
    RMS_GO(0);
  }
#undef RMS_GO
}

void launch_exit_gate(int dtype, const void* rows, int n_rows, int d, const void* w, float b, float* lam,
                      hipStream_t st) {
  if (n_rows <= 0) return;
  DISPATCH_T(dtype, T, k_exit_gate<T><<<n_rows, 256, 0, st>>>((const T*)rows, d, (const T*)w, b, lam));
}

void launch_qk_norm_rope(int dtype, const float* qkv, int n_rows, int rows_per_seq, int pos0, int Hq, int Hkv,
                         int hd, const void* qn, const void* kn, float eps, const float* cosT,
                         const float* sinT, void* q_out, void* k_out, void* v_out, int64_t kSeq, int64_t kHead,
                         int64_t kPos, int64_t vSeq, int64_t vHead, int64_t vRow, int seq0, hipStream_t st,
                         int splits, int kv_type) {
  if (n_rows <= 0) return;
  // q/k heads: one wave each; value heads: one block per (sequence, kv head, 64-position chunk)
  const int per_wave = n_rows >= 2048 ? 4 : 1;
  const int qk_blocks = (n_rows * (Hq + Hkv) + 4 * per_wave - 1) / (4 * per_wave);
  const int v_blocks = (n_rows / rows_per_seq) * Hkv * ((rows_per_seq + 63) / 64) * (hd / 32);
#define QKR_LAUNCH(T, TKV, S)                                                                             \
  if (per_wave == 4)                                                                                      \
    k_qk_norm_rope<T, T, TKV, S, 4><<<qk_blocks + v_blocks, 256, 0, st>>>(                                \
        qkv, n_rows, rows_per_seq, pos0, Hq, Hkv, hd, (const T*)qn, (const T*)kn, eps, cosT, sinT, (T*)q_out, \
        (TKV*)k_out, (TKV*)v_out, kSeq, kHead, kPos, vSeq, vHead, vRow, seq0, splits, qk_blocks);          \
  else                                                                                                    \
    k_qk_norm_rope<T, T, TKV, S, 1><<<qk_blocks + v_blocks, 256, 0, st>>>(                                \
        qkv, n_rows, rows_per_seq, pos0, Hq, Hkv, hd, (const T*)qn, (const T*)kn, eps, cosT, sinT, (T*)q_out, \
        (TKV*)k_out, (TKV*)v_out, kSeq, kHead, kPos, vSeq, vHead, vRow, seq0, splits, qk_blocks)
#define QKR_GO(S)                                   \
  if (kv_type == DT_FP8) {                          \
    QKR_LAUNCH(bf16_t, fp8_t, S);                   \
  } else {                                          \
    DISPATCH_T(dtype, T, QKR_LAUNCH(T, T, S));      \
  }
  if (splits <= 1) {
    QKR_GO(1);
  } else if (splits == 2) {
    QKR_GO(2);
  } else if (splits == 4) {
    QKR_GO(4);
  } else {
    QKR_GO(0);
  }
#undef QKR_GO
#undef QKR_LAUNCH
}

void launch_swiglu(int dtype, const float* gu, int n_rows, int F, void* act, hipStream_t st) {
  const size_t n = (size_t)n_rows * F;
  if (!n) return;
  DISPATCH_T(dtype, T, k_swiglu<T><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(gu, n_rows, F, (T*)act));
}

void launch_softstat_combine(const SoftStat* part, int n_rows, int n_tiles, const int32_t* n_dev, float* H,
                             float* lse, int32_t* tok, const GStat* gpart, int32_t* stok, hipStream_t st) {
  if (n_rows <= 0) return;
  k_softstat_combine<<<n_rows, 64, 0, st>>>(part, n_tiles, n_dev, H, lse, tok, gpart, stok);
}

void launch_step_init(const int32_t* block_ids, int B, int L, int mask_id, uint8_t* U, float* a,
                      int32_t* tokens, int8_t* cl, int32_t* ncommit, uint8_t* stop, int8_t* loops,
                      int32_t* act, int32_t* src_slot, hipStream_t st) {
  const int n = B * L;
  const int m = n > B ? n : B;
  k_step_init<<<(m + 255) / 256, 256, 0, st>>>(block_ids, n, mask_id, U, a, tokens, cl, B, ncommit, stop, loops,
                                               act, src_slot);
}

void launch_build_lists(int nb, int L, int B, int keep_all, const int32_t* act_cur, const uint8_t* stop,
                        const uint8_t* U,
                        const int32_t* ncommit, int32_t* act_next, int32_t* src_slot, int32_t* ro_rows,
                        int32_t* ro_map, int32_t* cnt, hipStream_t st) {
  k_build_lists<<<1, 1024, 0, st>>>(nb, L, B, keep_all, act_cur, stop, U, ncommit, act_next, src_slot, ro_rows,
                                     ro_map, cnt);
}

void launch_commit(int nb, int s, int k_loops, int L, int B, float tau_ent, float tau_halt, const int32_t* act,
                   uint8_t* U, float* a, const int32_t* ro_map, const float* H, const int32_t* tok,
                   const int32_t* stok, const float* lam, const float* lse, int32_t* tokens, int8_t* cl,
                   int32_t* ncommit, uint8_t* stop, int8_t* loops, const int8_t* tf_cl, const int32_t* tf_tok,
                   const int8_t* tf_stop, float* dbg_H, float* dbg_lam, float* dbg_a, float* dbg_lse,
                   int32_t* dbg_tok, int32_t* dbg_stok, hipStream_t st) {
  if (nb <= 0) return;
  k_commit<<<nb, 64, 0, st>>>(s, k_loops, L, B, tau_ent, tau_halt, act, U, a, ro_map, H, tok, stok, lam, lse,
                              tokens, cl, ncommit, stop, loops, tf_cl, tf_tok, tf_stop, dbg_H, dbg_lam, dbg_a,
                              dbg_lse, dbg_tok, dbg_stok);
}

void launch_reset_compact(int dtype, int nb_upper, const int32_t* cnt, int L, int d, int V, const int32_t* act,
                          const int32_t* src, const uint8_t* U, const int32_t* tokens, const float* h_old,
                          const void* E, float* h_new, hipStream_t st) {
  if (nb_upper <= 0) return;
  DISPATCH_T(dtype, T,
             k_reset_compact<T><<<nb_upper * L, 256, 0, st>>>(cnt, L, d, V, act, src, U, tokens, h_old, (const T*)E,
                                                              h_new));
}

void launch_dump_hidden(int nb, int L, int d, int B, int s, const int32_t* act, const float* h, float* out,
                        hipStream_t st) {
  if (nb <= 0) return;
  k_dump_hidden<<<nb * L, 256, 0, st>>>(nb, L, d, B, s, act, h, out);
}

void launch_gather_rows(const int32_t* ro_rows, const int32_t* n_dev, const int32_t* act, int n_upper, int L,
                        const int32_t* boost_tok, const float* boost_val, int32_t* btok, float* bval, int32_t* rkey,
                        hipStream_t st) {
  if (n_upper <= 0 || (!boost_tok && !rkey)) return;
  k_gather_rows<<<(n_upper + 255) / 256, 256, 0, st>>>(ro_rows, n_dev, act, n_upper, L, boost_tok, boost_val, btok,
                                                        bval, rkey);
}

void launch_block_init(const int32_t* block_ids, int n, int mask_id, int32_t* ids, int16_t* commit_step,
                       int8_t* commit_loop, int32_t* cnt, hipStream_t st) {
  k_block_init<<<1, 1024, 0, st>>>(block_ids, n, mask_id, ids, commit_step, commit_loop, cnt);
}

void launch_block_merge(int n, int t, const int32_t* step_tok, const int8_t* step_cl, int32_t* ids,
                        int16_t* commit_step, int8_t* commit_loop, hipStream_t st) {
  if (n > 0) k_block_merge<<<(n + 255) / 256, 256, 0, st>>>(n, t, step_tok, step_cl, ids, commit_step, commit_loop);
}

void launch_embed_committed(int dtype, const int8_t* cl, const int32_t* tokens, const void* E, int n, int d, int V,
                            float* out, hipStream_t st) {
  if (n <= 0) return;
  DISPATCH_T(dtype, T, k_embed_committed<T><<<n, 256, 0, st>>>(cl, tokens, (const T*)E, d, V, out));
}

}  // namespace alodlm
