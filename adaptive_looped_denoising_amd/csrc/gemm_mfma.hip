// bf16 GEMM on the gfx950 matrix cores: C[m][n] = sum_k A[m][k] B[n][k] with A, B row-major bf16
// (both K-contiguous), fp32 accumulation in v_mfma_f32_16x16x32_bf16.
//
// Block = 4 waves; tile BM x BN x 64 staged through LDS (double buffer, rows padded by 16 bytes
// so the 16-byte fragment reads of a wave hit distinct banks).  Tiles are numbered so that the
// blocks the dispatcher sends to one XCD (block ids congruent mod 8) are consecutive tiles with the
// row tile varying fastest: the few row tiles that share a weight column tile run on the same
// XCD at about the same time and find it in that XCD's L2.
//
// Epilogues: STORE (fp32), RESID (fp32 C = R + acc), SWIGLU (gate/up rows interleaved in
// 16-column groups, output bf16 silu(gate) * up), SOFTSTAT (per-row softmax statistics of the
// tile for the LM-head readout; logits never leave the chip).  Split-K writes fp32 partials
// that k_splitk_reduce sums in a fixed order and finishes with the same epilogue.
#include "common.h"
#include "launch.h"

namespace alodlm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int GK = 64;         // K per stage
constexpr int GLDK = GK + 8;   // LDS row pitch (bf16 elements)

// Row of B feeding column n of the (interleaved) gate/up product: 16-column groups alternate
// between gate rows p and up rows F + p, p = (n / 32) * 16 + n % 16.
__device__ __forceinline__ int swiglu_b_row(int n, int F) {
  const int p = (n >> 5) * 16 + (n & 15);
  return (n & 16) ? F + p : p;
}

template <int BM, int BN, int WM, int WN, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_mfma(const bf16_t* __restrict__ A, int lda,
                                                   const bf16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                   int k_split, int m_tiles, int n_tiles, int splits,
                                                   const int32_t* __restrict__ m_dev, GemmEpi ep, int F) {
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int A_CH = BM * (GK / 8), B_CH = BN * (GK / 8);
  constexpr int CH = (A_CH + B_CH) / 256;
  static_assert((A_CH + B_CH) % 256 == 0, "tile chunks must divide the block");
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * GLDK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * GLDK];

  // tile of this block (XCD-aware order, row tile fastest)
  const int total = m_tiles * n_tiles * splits;
  const int per = (gridDim.x + 7) >> 3;
  const int T = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (T >= total) return;
  const int mt = T % m_tiles;
  const int rest = T / m_tiles;
  const int nt = rest % n_tiles;
  const int sp = rest / n_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  int Mr = M;
  if (m_dev) Mr = min(Mr, *m_dev);
  if (m0 >= Mr) return;
  const int kb = sp * k_split;
  const int ke = min(K, kb + k_split);
  const int nk = (ke - kb) / GK;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int wm = wid / WN, wn = wid % WN;

  // per-thread global source of each 16-byte chunk (rows fixed across k)
  const bf16_t* src[CH];
  bool ok[CH];
  int soff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    int c = tid + i * 256;
    if (c < A_CH) {
      const int r = c >> 3, kc = (c & 7) * 8;
      const int gm = m0 + r;
      ok[i] = gm < Mr;
      src[i] = A + (size_t)(ok[i] ? gm : 0) * lda + kc;
      soff[i] = r * GLDK + kc;
    } else {
      c -= A_CH;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int gn = n0 + r;
      ok[i] = gn < N;
      const int brow = (EPI == EPI_SWIGLU) ? swiglu_b_row(ok[i] ? gn : 0, F) : (ok[i] ? gn : 0);
      src[i] = B + (size_t)brow * ldb + kc;
      soff[i] = -1 - (r * GLDK + kc);  // negative: B tile
    }
  }
  uint4 regs[CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) regs[i] = ok[i] ? *(const uint4*)(src[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (soff[i] >= 0)
        *(uint4*)&sA[buf][soff[i]] = regs[i];
      else
        *(uint4*)&sB[buf][-1 - soff[i]] = regs[i];
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (floatx4){0.f, 0.f, 0.f, 0.f};

  const int arow = wm * TM * 16 + (lane & 15);
  const int brow = wn * TN * 16 + (lane & 15);
  const int kq = (lane >> 4) * 8;

  if (nk > 0) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) gload(kb + (it + 1) * GK);
#pragma unroll
    for (int kk = 0; kk < GK; kk += 32) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) af[a] = *(const bf16x8_t*)&sA[buf][(arow + a * 16) * GLDK + kk + kq];
#pragma unroll
      for (int b = 0; b < TN; ++b) bfr[b] = *(const bf16x8_t*)&sB[buf][(brow + b * 16) * GLDK + kk + kq];
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
    if (it + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  const int rbase = m0 + wm * TM * 16 + 4 * (lane >> 4);
  const int cbase = n0 + wn * TN * 16 + (lane & 15);
  if (SPLIT) {
    float* P = ep.C + (size_t)sp * M * N;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = rbase + a * 16 + v;
        if (m >= Mr) continue;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int n = cbase + b * 16;
          if (n < N) P[(size_t)m * N + n] = acc[a][b][v];
        }
      }
    return;
  }
  if (EPI == EPI_STORE || EPI == EPI_RESID) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = rbase + a * 16 + v;
        if (m >= Mr) continue;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int n = cbase + b * 16;
          if (n >= N) continue;
          const size_t o = (size_t)m * ep.ldc + n;
          ep.C[o] = (EPI == EPI_RESID ? ep.R[o] : 0.f) + acc[a][b][v];
        }
      }
  } else if (EPI == EPI_SWIGLU) {
    bf16_t* act = (bf16_t*)ep.act;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = rbase + a * 16 + v;
        if (m >= Mr) continue;
#pragma unroll
        for (int b = 0; b < TN; b += 2) {
          const int n = cbase + b * 16;  // gate column (16-column group of even index)
          if (n >= N) continue;
          const int p = (n >> 5) * 16 + (n & 15);
          const float g = acc[a][b][v], u = acc[a][b + 1][v];
          act[(size_t)m * ep.ld_act + p] = from_f<bf16_t>(g / (1.0f + __expf(-g)) * u);
        }
      }
  } else if (EPI == EPI_SOFTSTAT) {
    __shared__ SoftStat red[WN][BM];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rl = wm * TM * 16 + a * 16 + 4 * (lane >> 4) + v;
        const int m = m0 + rl;
        const int bt = (m < Mr && ep.btok) ? ep.btok[m] : -1;
        const float bv = bt >= 0 ? ep.bval[m] : 0.f;
        SoftStat s = softstat_empty();
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int n = cbase + b * 16;
          if (n < N) {
            SoftStat e;
            e.m = acc[a][b][v] + (n == bt ? bv : 0.f);
            e.S = 1.f;
            e.T = 0.f;
            e.idx = n;
            s = softstat_merge(s, e);
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s = softstat_merge(s, softstat_shfl_xor(s, o));
        if ((lane & 15) == 0) red[wn][rl] = s;
      }
    __syncthreads();
    for (int rl = tid; rl < BM; rl += 256) {
      const int m = m0 + rl;
      if (m >= Mr) continue;
      SoftStat s = red[0][rl];
#pragma unroll
      for (int w = 1; w < WN; ++w) s = softstat_merge(s, red[w][rl]);
      ep.part[(size_t)m * ep.n_tiles + nt] = s;
    }
  }
}

// Fixed-order sum of split-K partials [splits][M][N] followed by the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int splits, int M, int N,
                                                       const int32_t* __restrict__ m_dev, GemmEpi ep) {
  int Mr = M;
  if (m_dev) Mr = min(Mr, *m_dev);
  const int NO = (EPI == EPI_SWIGLU) ? N / 2 : N;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)Mr * NO) return;
  const int m = (int)(i / NO), j = (int)(i % NO);
  if (EPI == EPI_SWIGLU) {
    const int ng = (j >> 4) * 32 + (j & 15);
    float g = 0.f, u = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float* P = part + (size_t)s * M * N + (size_t)m * N;
      g += P[ng];
      u += P[ng + 16];
    }
    ((bf16_t*)ep.act)[(size_t)m * ep.ld_act + j] = from_f<bf16_t>(g / (1.0f + __expf(-g)) * u);
  } else {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) acc += part[(size_t)s * M * N + (size_t)m * N + j];
    const size_t o = (size_t)m * ep.ldc + j;
    ep.C[o] = (EPI == EPI_RESID ? ep.R[o] : 0.f) + acc;
  }
}

// ---------------------------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
static void run_tile(int epi, bool split, dim3 grid, const bf16_t* A, int lda, const bf16_t* B, int ldb, int M,
                     int N, int K, int k_split, int mt, int nt, int splits, const int32_t* m_dev, const GemmEpi& ep,
                     int F, hipStream_t st) {
#define GO(E, S) \
  k_gemm_mfma<BM, BN, WM, WN, E, S><<<grid, 256, 0, st>>>(A, lda, B, ldb, M, N, K, k_split, mt, nt, splits, m_dev, ep, F)
  if (split) {
    if (epi == EPI_SWIGLU) GO(EPI_SWIGLU, true);
    else GO(EPI_STORE, true);
  } else if (epi == EPI_STORE) {
    GO(EPI_STORE, false);
  } else if (epi == EPI_RESID) {
    GO(EPI_RESID, false);
  } else if (epi == EPI_SWIGLU) {
    GO(EPI_SWIGLU, false);
  } else {
    GO(EPI_SOFTSTAT, false);
  }
#undef GO
}

bool gemm_mfma_supported(int K, int lda, int ldb) { return K % GK == 0 && lda % 8 == 0 && ldb % 8 == 0 && K > 0; }

int gemm_mfma_tile_n(int M) {
  (void)M;
  return 128;
}

// Chooses the tile and split-K, then launches.  For SWIGLU, N = 2F (interleaved gate/up columns)
// and the output has F columns.  part/part_floats: split-K scratch.
void launch_gemm_mfma(int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                      const int32_t* m_dev, const GemmEpi& ep, int F, float* part, size_t part_floats,
                      int force_splits, hipStream_t st) {
  if (M <= 0 || N <= 0) return;
  const int BM = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
  const int BN = 128;
  const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  int splits = 1;
  if (epi != EPI_SOFTSTAT) {
    if (force_splits > 0) {
      splits = force_splits;
    } else {
      while (mt * nt * splits < 512 && (K / GK) % (splits * 2) == 0 && K / (splits * 2) >= 512 &&
             (size_t)(splits * 2) * M * N <= part_floats)
        splits *= 2;
    }
    if ((size_t)splits * M * N > part_floats || (K / GK) % splits != 0) splits = 1;
  }
  const int k_split = K / splits;
  const int total = mt * nt * splits;
  const int per = (total + 7) / 8;
  dim3 grid(per * 8);
  const bool split = splits > 1;
  GemmEpi e = ep;
  if (split) {
    e.C = part;
    e.ldc = N;
  }
  const bf16_t* a = (const bf16_t*)A;
  const bf16_t* b = (const bf16_t*)B;
  if (BM == 32)
    run_tile<32, 128, 1, 4>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st);
  else if (BM == 64)
    run_tile<64, 128, 2, 2>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st);
  else
    run_tile<128, 128, 2, 2>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st);
  if (split) {
    const int NO = epi == EPI_SWIGLU ? N / 2 : N;
    const size_t n = (size_t)M * NO;
    const unsigned g = (unsigned)((n + 255) / 256);
    if (epi == EPI_SWIGLU)
      k_splitk_reduce<EPI_SWIGLU><<<g, 256, 0, st>>>(part, splits, M, N, m_dev, ep);
    else if (epi == EPI_RESID)
      k_splitk_reduce<EPI_RESID><<<g, 256, 0, st>>>(part, splits, M, N, m_dev, ep);
    else
      k_splitk_reduce<EPI_STORE><<<g, 256, 0, st>>>(part, splits, M, N, m_dev, ep);
  }
}

}  // namespace alodlm

#include "../../include/alodlm_diag.h"

extern "C" int alodlm_diag_gemm(int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, const void* B, float* C,
                                void* act, float* scratch, size_t scratch_floats, int32_t force_splits,
                                int32_t force_generic, void* hip_stream) {
  using namespace alodlm;
  if (M <= 0 || N <= 0 || K <= 0 || !A || !B) return -1;
  if (epi != EPI_STORE && epi != EPI_RESID && epi != EPI_SWIGLU) return -1;
  if (epi == EPI_SWIGLU && (!act || N % 32)) return -1;
  if (epi != EPI_SWIGLU && !C) return -1;
  if (force_splits > 1 && (!scratch || (size_t)force_splits * M * N > scratch_floats || (K / 64) % force_splits))
    return -1;
  hipStream_t st = (hipStream_t)hip_stream;
  GemmEpi ep;
  ep.C = C;
  ep.R = C;
  ep.ldc = N;
  ep.act = act;
  ep.ld_act = N / 2;
  if (force_generic || !gemm_mfma_supported(K, K, K)) {
    if (epi == EPI_SWIGLU) return -1;
    launch_gemm_generic(DT_BF16, epi, A, K, B, K, M, N, K, nullptr, ep, st);
  } else {
    launch_gemm_mfma(epi, A, K, B, K, M, N, K, nullptr, ep, N / 2, scratch, scratch ? scratch_floats : 0,
                     force_splits, st);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
