// Generic (any head size, fp32 or bf16 storage) GEMM and attention kernels.  They use the
// vector ALUs with fp32 arithmetic; the bf16 fast paths on the matrix cores live in
// gemm_mfma.hip and attn_mfma.hip.  These cover fp32 mode and every shape the fast
// paths do not.
#include "common.h"
#include "launch.h"

namespace alodlm {

// C[m][n] = sum_k A[m][k] B[n][k]; 64x64 output tile, 256 threads, 4x4 outputs per thread.
template <typename TA, typename TB, int EPI>
__global__ __launch_bounds__(256) void k_gemm_generic(const TA* __restrict__ A, int lda, const TB* __restrict__ B,
                                                      int ldb, int M, int N, int K,
                                                      const int32_t* __restrict__ m_dev, GemmEpi ep) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  int Mr = M;
  if (m_dev) Mr = min(Mr, *m_dev);
  if (m0 >= Mr) return;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int t = threadIdx.x; t < 1024; t += 256) {
      const int mm = t >> 4, kk = t & 15;
      const int gk = k0 + kk;
      const int gm = m0 + mm, gn = n0 + mm;
      As[kk][mm] = (gm < Mr && gk < K) ? to_f(A[(size_t)gm * lda + gk]) : 0.f;
      Bs[kk][mm] = (gn < N && gk < K) ? to_f(B[(size_t)gn * ldb + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  if (EPI == EPI_SOFTSTAT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + ty * 4 + i;
      const int bt = (m < Mr && ep.btok) ? ep.btok[m] : -1;
      const float bv = bt >= 0 ? ep.bval[m] : 0.f;
      SoftStat s = softstat_empty();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        if (n < N) {
          SoftStat e;
          e.m = acc[i][j] + (n == bt ? bv : 0.f);
          e.S = 1.f;
          e.T = 0.f;
          e.idx = n;
          s = softstat_merge(s, e);
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s = softstat_merge(s, softstat_shfl_xor(s, o));
      if (tx == 0 && m < Mr) ep.part[(size_t)m * ep.n_tiles + blockIdx.x] = s;
      if (ep.smp.part) {
        // this thread's four consecutive columns are the four words of one Philox block
        uint32_t c0 = (uint32_t)((n0 + tx * 4) >> 2), c1 = m < Mr ? (uint32_t)ep.smp.row_key[m] : 0u, c2 = ep.smp.c2,
                 c3 = ep.smp.c3;
        philox4x32_10(c0, c1, c2, c3, ep.smp.k0, ep.smp.k1);
        const uint32_t words[4] = {c0, c1, c2, c3};
        float gg = -INFINITY;
        int gi = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + tx * 4 + j;
          const float y = acc[i][j] + (n == bt ? bv : 0.f) + gumbel_of(words[j]);
          const bool tk = n < N && y > gg;
          gg = tk ? y : gg;
          gi = tk ? n : gi;
        }
        gstat_reduce_xor<8>(gg, gi);
        if (tx == 0 && m < Mr) ep.smp.part[(size_t)m * ep.n_tiles + blockIdx.x] = GStat{gg, gi};
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= Mr) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const size_t o = (size_t)m * ep.ldc + n;
      if (EPI == EPI_STORE)
        ep.C[o] = acc[i][j];
      else
        ep.C[o] = ep.R[o] + acc[i][j];
    }
  }
}

void launch_gemm_generic(int dtype, int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                         const int32_t* m_dev, const GemmEpi& ep, hipStream_t st) {
  if (M <= 0 || N <= 0) return;
  dim3 grid((N + 63) / 64, (M + 63) / 64);
#define GO(T, E) k_gemm_generic<T, T, E><<<grid, 256, 0, st>>>((const T*)A, lda, (const T*)B, ldb, M, N, K, m_dev, ep)
  if (dtype == DT_BF16) {
    if (epi == EPI_STORE) GO(bf16_t, EPI_STORE);
    else if (epi == EPI_RESID) GO(bf16_t, EPI_RESID);
    else GO(bf16_t, EPI_SOFTSTAT);
  } else {
    if (epi == EPI_STORE) GO(float, EPI_STORE);
    else if (epi == EPI_RESID) GO(float, EPI_RESID);
    else GO(float, EPI_SOFTSTAT);
  }
#undef GO
}

// ---------------------------------------------------------------------------------------------
// Attention of one query row and head per wave: keys are the prefix keys (the cache slot of the
// loop's depth plane) followed by the rows' own keys (all of them, or positions <= the query's
// when causal).  Online softmax over chunks of 64 keys: lane j scores key j, then every lane
// accumulates its head-dim elements.
template <typename T>
__device__ __forceinline__ const T* attn_k_ptr(const AttnParams& p, int j, int b, int t, int kvh) {
  if (j < p.n_cache) return (const T*)p.ck + (size_t)b * p.c_kSeq + (size_t)kvh * p.c_kHead + (size_t)j * p.c_kPos;
  const int jj = j - p.n_cache;
  return (const T*)p.sk + (size_t)(t + p.s_seq0) * p.s_kSeq + (size_t)kvh * p.s_kHead + (size_t)jj * p.s_kPos;
}
// element e of value j is at the returned pointer + e * (returned row stride)
template <typename T>
__device__ __forceinline__ const T* attn_v_ptr(const AttnParams& p, int j, int b, int t, int kvh, int64_t* row) {
  if (j < p.n_cache) {
    *row = p.c_vRow;
    return (const T*)p.cv + (size_t)b * p.c_vSeq + (size_t)kvh * p.c_vHead + j;
  }
  const int jj = j - p.n_cache;
  *row = p.s_vRow;
  return (const T*)p.sv + (size_t)(t + p.s_seq0) * p.s_vSeq + (size_t)kvh * p.s_vHead + jj;
}

template <typename T>
__global__ __launch_bounds__(64) void k_attn_generic(AttnParams p) {
  __shared__ float qs[128];
  const int lane = threadIdx.x;
  const int r = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
  const int kvh = (h * p.Hkv) / p.Hq;
  const int t = r / p.rows_per_seq, i = r % p.rows_per_seq;
  const int b = p.seq_map ? p.seq_map[t] : t;
  const T* q = (const T*)p.q + ((size_t)r * p.Hq + h) * p.hd;
  for (int e = lane; e < p.hd; e += 64) qs[e] = to_f(q[e]);
  __syncthreads();
  const int n_keys = p.n_cache + (p.causal ? min(i + 1 + p.causal_off, p.n_self) : p.n_self);
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int j0 = 0; j0 < n_keys; j0 += 64) {
    const int j = j0 + lane;
    float sc = -INFINITY;
    if (j < n_keys) {
      const T* kp = attn_k_ptr<T>(p, j, b, t, kvh);
      float dot = 0.f;
      for (int e = 0; e < p.hd; ++e) dot += qs[e] * to_f(kp[e]);
      sc = dot * p.scale;
    }
    const float mn = fmaxf(m, wave_max(sc));
    const float pj = (j < n_keys) ? __expf(sc - mn) : 0.f;
    const float corr = __expf(m - mn);
    l = l * corr + wave_sum(pj);
    acc0 *= corr;
    acc1 *= corr;
    const int nk = min(64, n_keys - j0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pw = __shfl(pj, jj, 64);
      int64_t vr;
      const T* vp = attn_v_ptr<T>(p, j0 + jj, b, t, kvh, &vr);
      if (lane < p.hd) acc0 += pw * to_f(vp[(size_t)lane * vr]);
      if (lane + 64 < p.hd) acc1 += pw * to_f(vp[(size_t)(lane + 64) * vr]);
    }
    m = mn;
  }
  T* o = (T*)p.out + (size_t)r * p.Hq * p.hd + (size_t)h * p.hd;
  const float inv = 1.0f / l;
  if (lane < p.hd) o[lane] = from_f<T>(acc0 * inv);
  if (lane + 64 < p.hd) o[lane + 64] = from_f<T>(acc1 * inv);
}

void launch_attn_generic(int dtype, const AttnParams& p, hipStream_t st) {
  if (p.n_rows <= 0) return;
  if (dtype == DT_BF16)
    k_attn_generic<bf16_t><<<p.n_rows * p.Hq, 64, 0, st>>>(p);
  else
    k_attn_generic<float><<<p.n_rows * p.Hq, 64, 0, st>>>(p);
}

}  // namespace alodlm
