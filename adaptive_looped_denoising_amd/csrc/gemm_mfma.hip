// bf16 GEMM on the gfx950 matrix cores: C[m][n] = sum_k A[m][k] B[n][k] with A, B row-major bf16
// (both K-contiguous), fp32 accumulation in v_mfma_f32_16x16x32_bf16.
//
// Kernel families (tile table kTiles, chosen per shape by gemm_mfma_auto_tile):
//   k_gemm_mfma   4 waves, BM x BN x 64 tiles double-buffered through padded LDS rows;
//   k_gemm_pipe   4 or 8 waves (two per SIMD), an NS-stage LDS ring filled by direct
//                 global->LDS loads with XOR-swizzled 16-byte chunks, explicit vmcnt waits;
//   k_gemm_adirect activations straight to registers, weights through the LDS ring;
//   k_gemm_ring2  separate activation / weight ring depths;
//   k_gemm_ws     wave-specialised loads (half the waves fetch activations, half weights);
//   k_gemm_wide   eight 64-row waves over 256-row tiles, 32-deep stages, each stage's fragments
//                 read while the matrix cores work on the previous one; for many rows the
//                 dispatcher now takes the pipelined 256 x 256 tile with two 64-deep stages,
//                 which runs the same MFMAs in the same order and measured faster.
// Tiles are numbered so that the blocks the dispatcher sends to one XCD (block ids congruent
// mod 8) are consecutive tiles with the row tile varying fastest: the few row tiles that share
// a weight column tile run on the same XCD at about the same time and find it in its L2.
//
// Epilogues: STORE (fp32), RESID (fp32 C = R + acc), SWIGLU (gate/up rows interleaved in
// 16-column groups, output bf16 silu(gate) * up), SOFTSTAT (per-row softmax statistics of the
// tile for the LM-head readout, optionally with the Gumbel-max draw; logits never leave the
// chip).  Split-K writes fp32 partials that k_splitk_reduce sums in a fixed order and finishes
// with the same epilogue, or that the consuming kernel sums (deferred reduction).
#include <stdio.h>

#include <type_traits>

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
__device__ __forceinline__ void gemm_epilogue(floatx4 (&acc)[BM / WM / 16][BN / WN / 16], int m0, int n0, int nt,
                                              int sp, int Mr, int M, int N, const GemmEpi& ep, int wm, int wn,
                                              int lane, int tid, SoftStat* red) {
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
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
    // red (WN * BM entries) lives in the kernel's own operand LDS, reused once every wave is
    // past its last fragment read: a second LDS object would make the compiler's tracking of
    // the direct global->LDS loads wait for all of them before every fragment read of the loop.
    // With sampling, gred (WN * BM draws) follows red in the same LDS.
    GStat* gred = (GStat*)(red + WN * BM);
    const bool smp = ep.smp.part != nullptr;
    __syncthreads();
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rl = wm * TM * 16 + a * 16 + 4 * (lane >> 4) + v;
        const int m = m0 + rl;
        const int bt = (m < Mr && ep.btok) ? ep.btok[m] : -1;
        const float bv = bt >= 0 ? ep.bval[m] : 0.f;
        // this lane's TN logits of the row: max (first column attaining it), then
        // S = sum exp(z - max) and T = sum (z - max) exp(z - max), one exponential per logit
        float z[TN];
        float mx = -INFINITY;
        int ix = 0x7FFFFFFF;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int n = cbase + b * 16;
          z[b] = n < N ? acc[a][b][v] + (n + ep.col0 == bt ? bv : 0.f) : -INFINITY;
          if (z[b] > mx) {
            mx = z[b];
            ix = n + ep.col0;
          }
        }
        SoftStat s = softstat_empty();
        if (ix != 0x7FFFFFFF) {
          float S = 0.f, Tt = 0.f;
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const float dz = z[b] - mx;
            const float e = __expf(dz);  // exp(-inf) = 0 for columns past N
            S += e;
            Tt += z[b] > -INFINITY ? dz * e : 0.f;
          }
          s.m = mx;
          s.S = S;
          s.T = Tt;
          s.idx = ix;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s = softstat_merge(s, softstat_shfl_xor(s, o));
        if ((lane & 15) == 0) red[wn * BM + rl] = s;
      }
    }
    if (smp) {
      // Gumbel-max draws, one 16-row block at a time (few extra registers beside the
      // accumulators): lane q of each group of four lanes (four consecutive columns, the same four
      // rows) draws one Philox block for row q, i.e. that row's noise of the four columns; a 4x4
      // transpose over the group hands every lane its own column's noise for its four rows.
      const int q = lane & 3;
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int r0 = m0 + wm * TM * 16 + a * 16 + 4 * (lane >> 4);
        const uint32_t rk = r0 + q < Mr ? (uint32_t)ep.smp.row_key[r0 + q] : 0u;
        int btv[4];
        float bvv[4], gg[4];
        int gi[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          btv[v] = (r0 + v < Mr && ep.btok) ? ep.btok[r0 + v] : -1;
          bvv[v] = btv[v] >= 0 ? ep.bval[r0 + v] : 0.f;
          gg[v] = -INFINITY;
          gi[v] = 0x7FFFFFFF;
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          uint32_t c0 = (uint32_t)((ep.col0 + n0 + wn * TN * 16 + b * 16 + (lane & 12)) >> 2), c1 = rk, c2 = ep.smp.c2,
                   c3 = ep.smp.c3;
          philox4x32_10(c0, c1, c2, c3, ep.smp.k0, ep.smp.k1);
          float g[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            // round k: every lane sends its word (q + k) mod 4 and receives, from the lane that drew
            // row (q - k) mod 4, that row's word q (this lane's column)
            const int sw = (q + k) & 3;
            const uint32_t w = (sw & 2) ? ((sw & 1) ? c3 : c2) : ((sw & 1) ? c1 : c0);
            const uint32_t got = k == 0 ? w : (uint32_t)__shfl((int)w, (lane & ~3) | ((q - k) & 3), 64);
            const float gv = gumbel_of(got);
            const int row = (q - k) & 3;
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (row == v) g[v] = gv;
          }
          const int n = cbase + b * 16;  // ascending over b, so ties keep the lowest column
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float y = acc[a][b][v] + (n + ep.col0 == btv[v] ? bvv[v] : 0.f) + g[v];
            const bool tk = n < N && y > gg[v];
            gg[v] = tk ? y : gg[v];
            gi[v] = tk ? n + ep.col0 : gi[v];
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          gstat_reduce_xor<8>(gg[v], gi[v]);
          if ((lane & 15) == 0) gred[wn * BM + wm * TM * 16 + a * 16 + 4 * (lane >> 4) + v] = GStat{gg[v], gi[v]};
        }
      }
    }
    __syncthreads();
    for (int rl = tid; rl < BM; rl += 256) {
      const int m = m0 + rl;
      if (m >= Mr) continue;
      SoftStat s = red[rl];
#pragma unroll
      for (int w = 1; w < WN; ++w) s = softstat_merge(s, red[w * BM + rl]);
      ep.part[(size_t)m * ep.n_tiles + nt] = s;
      if (smp) {
        float gg = gred[rl].g;
        int gi = gred[rl].idx;
#pragma unroll
        for (int w = 1; w < WN; ++w) gstat_take(gg, gi, gred[w * BM + rl].g, gred[w * BM + rl].idx);
        ep.smp.part[(size_t)m * ep.n_tiles + nt] = GStat{gg, gi};
      }
    }
  }
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
  static_assert(WM * WN == 4 && TM * WM * 16 == BM && TN * WN * 16 == BN, "wave grid must tile the block");
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

  gemm_epilogue<BM, BN, WM, WN, EPI, SPLIT>(acc, m0, n0, nt, sp, Mr, M, N, ep, wm, wn, lane, tid, (SoftStat*)&sA[0][0]);
}

// Pipelined variant: an NS-stage LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane, so one wave instruction
// fills 8 consecutive 128-byte tile rows).  Up to NS-1 stages are in flight while the matrix cores
// work on the oldest one.  Row r of a stage keeps its eight 16-byte k-chunks XOR-swizzled
// (chunk c at slot c ^ (r & 7)) so that the 16 rows a fragment read touches spread over the banks.
// Rows past M / N load row 0 (never stored).

// Grouped tile order for many row tiles: consecutive tile numbers walk GM row tiles, then the
// next column tile, so the 32 workgroups an XCD holds at a time cover GM row panels and 32/GM
// column panels (12 distinct panels for GM = 8) instead of 32 row panels and one column panel:
// each panel's K-slice is then read from the XCD's L2 by several workgroups rather than from
// the memory-side cache by one.  With fewer than GM row tiles this is the plain row-fastest order.
__device__ __forceinline__ void grouped_tile(int T, int m_tiles, int n_tiles, int& mt, int& nt, int& sp) {
  constexpr int GM = 8;
  const int mn = m_tiles * n_tiles;
  sp = T / mn;
  const int t = T % mn;
  const int group = t / (GM * n_tiles);
  const int first = group * GM;
  const int gm = min(m_tiles - first, GM);
  const int w = t % (GM * n_tiles);
  mt = first + w % gm;
  nt = w / gm;
}

// WM x WN waves (4 or 8; with 8, two waves share each SIMD and hide each other's waits).
template <int BM, int BN, int WM, int WN, int NS, int EPI, bool SPLIT>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_pipe(const bf16_t* __restrict__ A, int lda,
                                                            const bf16_t* __restrict__ B, int ldb, int M, int N,
                                                            int K, int k_split, int m_tiles, int n_tiles, int splits,
                                                            const int32_t* __restrict__ m_dev, GemmEpi ep, int F) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int ROWS = BM + BN;                 // 128-byte rows per stage
  constexpr int STAGE = ROWS * 64;              // bf16 elements per stage
  constexpr int LPW = ROWS / (8 * NW);          // load instructions per wave per stage
  static_assert(ROWS % (8 * NW) == 0, "stage rows must split over the waves x 8 rows");
  static_assert((NW == 4 || NW == 8) && TM * WM * 16 == BM && TN * WN * 16 == BN, "wave grid must tile the block");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NS * STAGE];

  const int total = m_tiles * n_tiles * splits;
  const int per = (gridDim.x + 7) >> 3;
  const int T = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (T >= total) return;
  int mt, nt, sp;
  grouped_tile(T, m_tiles, n_tiles, mt, nt, sp);
  const int m0 = mt * BM, n0 = nt * BN;
  int Mr = M;
  if (m_dev) Mr = min(Mr, *m_dev);
  if (m0 >= Mr) return;
  const int kb = sp * k_split;
  const int nk = (min(K, kb + k_split) - kb) / GK;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int wm = wid / WN, wn = wid % WN;

  // this lane's global source row and k-chunk for each of its LPW load instructions
  const bf16_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int rho = (wid * LPW + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (rho & 7);
    if (rho < BM) {
      const int gm = m0 + rho;
      src[j] = A + (size_t)(gm < Mr ? gm : 0) * lda + c * 8;
    } else {
      const int gn = n0 + rho - BM;
      const int ok = gn < N ? gn : 0;
      const int brow = (EPI == EPI_SWIGLU) ? swiglu_b_row(ok, F) : ok;
      src[j] = B + (size_t)brow * ldb + c * 8;
    }
  }
  auto issue = [&](int stage_k, int slot) {
    bf16_t* base = smem + slot * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + stage_k), LDS_PTR(base + (wid * LPW + j) * 8 * 64), 16,
                                       0, 0);
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (floatx4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(kb + s * GK, s);

  const int col = lane & 15, quad = lane >> 4;
  for (int it = 0; it < nk; ++it) {
    if (it + NS - 1 <= nk)
      wait_vmcnt_le<(NS - 2) * LPW>();
    else
      wait_vmcnt_le<0>();
    // Workgroup barrier without the release/acquire fence __syncthreads() carries (the fence
    // would wait for every load in flight).  This wave's stage-`it` loads are complete (waitcnt
    // above); after the barrier so are every other wave's, and all reads of the slot refilled
    // below finished in the previous iteration.  The empty asm keeps the compiler from moving
    // LDS accesses across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + NS - 1 < nk) issue(kb + (it + NS - 1) * GK, (it + NS - 1) % NS);
    const bf16_t* st = smem + (it % NS) * STAGE;
    // all fragment reads of the stage first, so the second k-chunk's reads overlap the first
    // chunk's matrix-core work
    bf16x8_t af[2][TM], bfr[2][TN];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int c = kc * 4 + quad;
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int r = wm * TM * 16 + a * 16 + col;
        af[kc][a] = *(const bf16x8_t*)&st[r * 64 + ((c ^ (r & 7)) << 3)];
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int r = BM + wn * TN * 16 + b * 16 + col;
        bfr[kc][b] = *(const bf16x8_t*)&st[r * 64 + ((c ^ (r & 7)) << 3)];
      }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kc][a], bfr[kc][b], acc[a][b], 0, 0, 0);
  }
  gemm_epilogue<BM, BN, WM, WN, EPI, SPLIT>(acc, m0, n0, nt, sp, Mr, M, N, ep, wm, wn, lane, tid, (SoftStat*)smem);
}

// Wide tiles for many rows (prefill, long-context steps), where the matrix cores rather than the
// weight stream bound the GEMM (kept in the tile table; the dispatcher prefers the pipelined
// 256 x 256 tile, whose 64-deep stages bring each row's whole 128-byte line at once).  Eight waves hold 64 x (BN / 2) accumulator tiles each, so every
// 16-byte fragment read from LDS feeds (TM * TN) / (TM + TN) MFMAs, about twice the reuse of the
// 128-row tiles.  Stages are 32 deep in K (64-byte rows, four 16-byte chunks, chunk c of row r at
// slot c ^ ((r >> 1) & 3): the LDS serves a 16-byte read eight lanes at a time over 128 bytes of
// banks, i.e. two 64-byte rows, and the eight consecutive rows those lanes read (same chunk) then
// land in eight distinct 16-byte bank groups -- swizzling by r >> 2 instead left rows r and r + 2
// on the same banks: half of the LDS-active cycles were bank conflicts in rocprofv3), so
// NS stages of a 256 x 256 tile fit in LDS with NS - 2 stages of load latency cover.  Each
// stage's fragments are read into one of two register sets while the matrix cores work on the
// other stage's; the reads are retired with explicit LDS-counter waits one stage later (the
// compiler's own waits treat the direct-to-LDS loads as unordered with the fragment reads and
// would wait for the reads just issued as well).  The stage requested in iteration it
// overwrites the slot of stage it - 1, whose fragments every wave has retired before arriving
// at iteration it's barrier.
constexpr int WK = 32;  // K per stage of the wide tiles

template <int BM, int BN, int WM, int WN, int NS, int EPI, bool SPLIT>
__device__ __forceinline__ void gemm_wide_body(const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B,
                                               int ldb, int M, int N, int K, int k_split, int m_tiles, int n_tiles,
                                               int splits, const int32_t* __restrict__ m_dev, const GemmEpi& ep,
                                               int F, bf16_t* smem) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int ROWS = BM + BN;                 // 64-byte rows per stage
  constexpr int STAGE = ROWS * WK;              // bf16 elements per stage
  constexpr int LPW = ROWS / (16 * NW);         // load instructions per wave per stage
  static_assert(TM * WM * 16 == BM && TN * WN * 16 == BN && ROWS % (16 * NW) == 0, "waves must tile the block");
  static_assert(NS >= 3, "fragment prefetch needs three or more stages");

  const int total = m_tiles * n_tiles * splits;
  const int per = (gridDim.x + 7) >> 3;
  const int T = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (T >= total) return;
  int mt, nt, sp;
  grouped_tile(T, m_tiles, n_tiles, mt, nt, sp);
  const int m0 = mt * BM, n0 = nt * BN;
  int Mr = M;
  if (m_dev) Mr = min(Mr, *m_dev);
  if (m0 >= Mr) return;
  const int kb = sp * k_split;
  const int nk = (min(K, kb + k_split) - kb) / WK;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int wm = wid / WN, wn = wid % WN;

  // load instruction j of this wave fills stage rows (wid * LPW + j) * 16 .. + 15; this lane's
  // 16 bytes land at row rho, slot lane & 3, and hold global chunk (lane & 3) ^ ((rho >> 1) & 3)
  const bf16_t* src[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int rho = (wid * LPW + j) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((rho >> 1) & 3);
    if (rho < BM) {
      const int gm = m0 + rho;
      src[j] = A + (size_t)(gm < Mr ? gm : 0) * lda + c * 8;
    } else {
      const int gn = n0 + rho - BM;
      const int ok = gn < N ? gn : 0;
      const int brow = (EPI == EPI_SWIGLU) ? swiglu_b_row(ok, F) : ok;
      src[j] = B + (size_t)brow * ldb + c * 8;
    }
  }
  auto issue = [&](int stage_k, int slot) {
    bf16_t* base = smem + slot * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + stage_k), LDS_PTR(base + (wid * LPW + j) * 16 * WK), 16,
                                       0, 0);
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (floatx4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(kb + s * WK, s);

  const int col = lane & 15, quad = lane >> 4;
  auto read = [&](int slot, bf16x8_t (&fa)[TM], bf16x8_t (&fb)[TN]) {
    const bf16_t* st = smem + slot * STAGE;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int r = wm * TM * 16 + a * 16 + col;
      fa[a] = *(const bf16x8_t*)&st[r * WK + ((quad ^ ((r >> 1) & 3)) << 3)];
    }
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int r = BM + wn * TN * 16 + b * 16 + col;
      fb[b] = *(const bf16x8_t*)&st[r * WK + ((quad ^ ((r >> 1) & 3)) << 3)];
    }
  };
  auto mma = [&](bf16x8_t (&fa)[TM], bf16x8_t (&fb)[TN]) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
  };
  // Iteration it: make stage it + 1 visible, request stage it + NS - 1, retire stage it's
  // fragment reads, read stage it + 1's into the other register set (unconditionally: in the
  // last iteration the slot read is one no load writes any more, into registers nobody uses),
  // then multiply stage it.
  auto step = [&](int it, bf16x8_t (&ca)[TM], bf16x8_t (&cb)[TN], bf16x8_t (&na)[TM], bf16x8_t (&nb)[TN]) {
    if (it + 1 < nk) {
      if (it + NS - 2 <= nk - 1)
        wait_vmcnt_le<(NS - 3) * LPW>();
      else
        wait_vmcnt_le<0>();
      lds_barrier();
      if (it + NS - 1 < nk) issue(kb + (it + NS - 1) * WK, (it + NS - 1) % NS);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    read((it + 1) % NS, na, nb);
    __builtin_amdgcn_sched_barrier(0);
    mma(ca, cb);
    __builtin_amdgcn_sched_barrier(0);
  };

  bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  if (nk > 0) {
    if (NS - 2 <= nk - 1)
      wait_vmcnt_le<(NS - 2) * LPW>();
    else
      wait_vmcnt_le<0>();
    lds_barrier();
    read(0, fa0, fb0);
  }
  for (int it = 0; it < nk; it += 2) {
    step(it, fa0, fb0, fa1, fb1);
    if (it + 1 < nk) step(it + 1, fa1, fb1, fa0, fb0);
  }
  gemm_epilogue<BM, BN, WM, WN, EPI, SPLIT>(acc, m0, n0, nt, sp, Mr, M, N, ep, wm, wn, lane, tid, (SoftStat*)smem);
}

// Eight waves (two per SIMD), 64-row wave tiles.
template <int BM, int BN, int NS, int EPI, bool SPLIT>
__global__ __launch_bounds__(512) void k_gemm_wide(const bf16_t* __restrict__ A, int lda,
                                                   const bf16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                   int k_split, int m_tiles, int n_tiles, int splits,
                                                   const int32_t* __restrict__ m_dev, GemmEpi ep, int F) {
  constexpr int WM = BM / 64;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NS * (BM + BN) * WK];
  gemm_wide_body<BM, BN, WM, 8 / WM, NS, EPI, SPLIT>(A, lda, B, ldb, M, N, K, k_split, m_tiles, n_tiles, splits,
                                                     m_dev, ep, F, smem);
}

// Dual-ring variant: the activation tile (re-read by every column tile, so it comes from L2) and
// the weight tile (read once, from HBM) have LDS rings of their own, DA + 1 and DB + 1 stages
// deep, with DB > DA: weight stages are requested DB iterations ahead, activation stages DA
// ahead, so more HBM bytes are in flight per compute unit than one shared ring of the same LDS
// size allows.  Issue order is uniform over virtual iterations j = -DB .. nk - 1: A(j + DA) then
// B(j + DB), each only if its stage exists; the wait before iteration `it` counts exactly the
// loads issued after A(it) (the later of the two loads that iteration needs).
template <int LA, int LB, int DA, int CA = 0, int CB = 0>
__device__ __forceinline__ void ring2_wait(int ca, int cb) {
  if (ca == CA && cb == CB) {
    wait_vmcnt_le<CA * LA + CB * LB>();
    return;
  }
  if constexpr (CB < DA)
    ring2_wait<LA, LB, DA, CA, CB + 1>(ca, cb);
  else if constexpr (CA < DA - 1)
    ring2_wait<LA, LB, DA, CA + 1, 0>(ca, cb);
  else
    wait_vmcnt_le<0>();
}

template <int BM, int BN, int WM, int WN, int DA, int DB, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_ring2(const bf16_t* __restrict__ A, int lda,
                                                    const bf16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                    int k_split, int m_tiles, int n_tiles, int splits,
                                                    const int32_t* __restrict__ m_dev, GemmEpi ep, int F) {
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int LA = BM / 32, LB = BN / 32;     // load instructions per wave per stage
  constexpr int SA = BM * 64, SB = BN * 64;     // bf16 elements per stage
  static_assert(BM % 32 == 0 && BN % 32 == 0 && DA >= 1 && DB > DA, "ring shape (B of a stage is issued before its A)");
  static_assert(WM * WN == 4 && TM * WM * 16 == BM && TN * WN * 16 == BN, "wave grid must tile the block");
  // one LDS object for both rings: with two, the compiler's LDS-DMA tracking inserts a full
  // vector-memory wait before the fragment reads of the second
  __shared__ __attribute__((aligned(1024))) bf16_t smem[(DA + 1) * SA + (DB + 1) * SB];
  bf16_t* const sa = smem;
  bf16_t* const sb = smem + (DA + 1) * SA;

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
  const int nk = (min(K, kb + k_split) - kb) / GK;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int wm = wid / WN, wn = wid % WN;

  const bf16_t* asrc[LA];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int rho = (wid * LA + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (rho & 7);
    const int gm = m0 + rho;
    asrc[j] = A + (size_t)(gm < Mr ? gm : 0) * lda + c * 8;
  }
  const bf16_t* bsrc[LB];
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int rho = (wid * LB + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (rho & 7);
    const int gn = n0 + rho;
    const int ok = gn < N ? gn : 0;
    const int brow = (EPI == EPI_SWIGLU) ? swiglu_b_row(ok, F) : ok;
    bsrc[j] = B + (size_t)brow * ldb + c * 8;
  }
  auto issue = [&](int j) {  // virtual iteration j: A(j + DA), then B(j + DB)
    const int xa = j + DA, xb = j + DB;
    if (xa >= 0 && xa < nk) {
      bf16_t* base = sa + (xa % (DA + 1)) * SA;
      const int k = kb + xa * GK;
#pragma unroll
      for (int i = 0; i < LA; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + k), LDS_PTR(base + (wid * LA + i) * 8 * 64), 16, 0, 0);
    }
    if (xb < nk) {
      bf16_t* base = sb + (xb % (DB + 1)) * SB;
      const int k = kb + xb * GK;
#pragma unroll
      for (int i = 0; i < LB; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + k), LDS_PTR(base + (wid * LB + i) * 8 * 64), 16, 0, 0);
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (floatx4){0.f, 0.f, 0.f, 0.f};

  for (int j = -DB; j < 0; ++j) issue(j);

  const int col = lane & 15, quad = lane >> 4;
  for (int it = 0; it < nk; ++it) {
    // loads issued after A(it): B of virtual iterations it-DA .. it-1 and A of it-DA+1 .. it-1
    const int cb = min(max(nk - DB - (it - DA), 0), DA);
    const int ca = min(max(nk - 1 - it, 0), DA - 1);
    if (ca == DA - 1 && cb == DA)
      wait_vmcnt_le<(DA - 1) * LA + DA * LB>();
    else
      ring2_wait<LA, LB, DA>(ca, cb);
    // barrier without the fence of __syncthreads (see k_gemm_pipe): stage `it` has landed for
    // every wave, and every wave is done reading the slots refilled by issue(it) below.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(it);
    const bf16_t* ta = sa + (it % (DA + 1)) * SA;
    const bf16_t* tb = sb + (it % (DB + 1)) * SB;
    bf16x8_t af[2][TM], bfr[2][TN];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int c = kc * 4 + quad;
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int r = wm * TM * 16 + a * 16 + col;
        af[kc][a] = *(const bf16x8_t*)&ta[r * 64 + ((c ^ (r & 7)) << 3)];
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int r = wn * TN * 16 + b * 16 + col;
        bfr[kc][b] = *(const bf16x8_t*)&tb[r * 64 + ((c ^ (r & 7)) << 3)];
      }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kc][a], bfr[kc][b], acc[a][b], 0, 0, 0);
  }
  gemm_epilogue<BM, BN, WM, WN, EPI, SPLIT>(acc, m0, n0, nt, sp, Mr, M, N, ep, wm, wn, lane, tid, (SoftStat*)smem);
}

// Wave-specialised loads: eight waves all compute, but the first half of them fetch only the
// activation tile (from L2, DA stages ahead) and the second half only the weight tile (from HBM,
// DB stages ahead).  vmcnt counts a wave's own loads in issue order, so when one wave fetches
// both streams, waiting for a near activation stage also waits for every weight load issued
// before it; with one stream per wave each wave waits only on its own, and the weight stream
// keeps DB stages of HBM latency in flight.
// vmcnt <= c * L for the runtime count c in 0 .. D-1 (immediate forms)
template <int L, int D, int C = 0>
__device__ __forceinline__ void wait_stream(int c) {
  if (c == C) {
    wait_vmcnt_le<C * L>();
    return;
  }
  if constexpr (C + 1 < D) wait_stream<L, D, C + 1>(c);
  else wait_vmcnt_le<0>();
}

template <int BM, int BN, int WM, int WN, int DA, int DB, int EPI, bool SPLIT>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_ws(const bf16_t* __restrict__ A, int lda,
                                                          const bf16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                          int k_split, int m_tiles, int n_tiles, int splits,
                                                          const int32_t* __restrict__ m_dev, GemmEpi ep, int F) {
  constexpr int NW = WM * WN;
  constexpr int HW = NW / 2;                    // waves per stream
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int LA = BM / (8 * HW), LB = BN / (8 * HW);  // load instructions per loading wave per stage
  constexpr int SA = BM * 64, SB = BN * 64;
  static_assert(NW == 8 && BM % (8 * HW) == 0 && BN % (8 * HW) == 0 && DA >= 1 && DB >= 1, "shape");
  static_assert(TM * WM * 16 == BM && TN * WN * 16 == BN, "wave grid must tile the block");
  static_assert((DA - 1) * LA < 64 && (DB - 1) * LB < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[(DA + 1) * SA + (DB + 1) * SB];
  bf16_t* const sa = smem;
  bf16_t* const sb = smem + (DA + 1) * SA;

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
  const int nk = (min(K, kb + k_split) - kb) / GK;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int wm = wid / WN, wn = wid % WN;
  const bool a_wave = wid < HW;
  const int lw = a_wave ? wid : wid - HW;       // index among the waves of this stream

  constexpr int LMAX = LA > LB ? LA : LB;
  const bf16_t* src[LMAX];
#pragma unroll
  for (int j = 0; j < LMAX; ++j) {
    if (a_wave) {
      const int rho = (lw * LA + (j < LA ? j : 0)) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ (rho & 7);
      const int gm = m0 + rho;
      src[j] = A + (size_t)(gm < Mr ? gm : 0) * lda + c * 8;
    } else {
      const int rho = (lw * LB + (j < LB ? j : 0)) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ (rho & 7);
      const int gn = n0 + rho;
      const int ok = gn < N ? gn : 0;
      const int brow = (EPI == EPI_SWIGLU) ? swiglu_b_row(ok, F) : ok;
      src[j] = B + (size_t)brow * ldb + c * 8;
    }
  }
  auto issue = [&](int stage) {  // this wave's share of its stream for k-stage `stage`
    const int k = kb + stage * GK;
    if (a_wave) {
      bf16_t* base = sa + (stage % (DA + 1)) * SA;
#pragma unroll
      for (int j = 0; j < LA; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src[j] + k), LDS_PTR(base + (lw * LA + j) * 512), 16, 0, 0);
    } else {
      bf16_t* base = sb + (stage % (DB + 1)) * SB;
#pragma unroll
      for (int j = 0; j < LB; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src[j] + k), LDS_PTR(base + (lw * LB + j) * 512), 16, 0, 0);
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (floatx4){0.f, 0.f, 0.f, 0.f};

  const int depth = a_wave ? DA : DB;
  for (int s = 0; s < depth && s < nk; ++s) issue(s);

  const int col = lane & 15, quad = lane >> 4;
  for (int it = 0; it < nk; ++it) {
    // own loads issued after stage `it`: stages it+1 .. min(it+depth-1, nk-1)
    const int c = min(max(nk - 1 - it, 0), depth - 1);
    if (a_wave) {
      if (c == DA - 1) wait_vmcnt_le<(DA - 1) * LA>();
      else wait_stream<LA, DA>(c);
    } else {
      if (c == DB - 1) wait_vmcnt_le<(DB - 1) * LB>();
      else wait_stream<LB, DB>(c);
    }
    // every wave's share of stage `it` has landed; every wave is done with stage it-1, whose
    // slots the issue below refills
    lds_barrier();
    if (it + depth < nk) issue(it + depth);
    const bf16_t* ta = sa + (it % (DA + 1)) * SA;
    const bf16_t* tb = sb + (it % (DB + 1)) * SB;
    bf16x8_t af[2][TM], bfr[2][TN];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int cc = kc * 4 + quad;
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int r = wm * TM * 16 + a * 16 + col;
        af[kc][a] = *(const bf16x8_t*)&ta[r * 64 + ((cc ^ (r & 7)) << 3)];
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int r = wn * TN * 16 + b * 16 + col;
        bfr[kc][b] = *(const bf16x8_t*)&tb[r * 64 + ((cc ^ (r & 7)) << 3)];
      }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kc][a], bfr[kc][b], acc[a][b], 0, 0, 0);
  }
  gemm_epilogue<BM, BN, WM, WN, EPI, SPLIT>(acc, m0, n0, nt, sp, Mr, M, N, ep, wm, wn, lane, tid, (SoftStat*)smem);
}

// Weight-streaming variant for 65..256 rows: the four waves split the 256 rows (64 each) and all
// read the same BN weight columns.  Only the shared weight tile goes through LDS (an NS-stage
// ring of direct global->LDS loads); each wave fetches its own activation fragments straight into
// registers in the matrix-core operand layout, two stages ahead (they hit L2: every column tile
// of the GEMM re-reads the same <= 2 MB of activations).  LDS traffic per stage is the weight
// tile written once and read by four waves.
template <int BN, int NS, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_adirect(const bf16_t* __restrict__ A, int lda,
                                                      const bf16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                      int k_split, int m_tiles, int n_tiles, int splits,
                                                      const int32_t* __restrict__ m_dev, GemmEpi ep, int F) {
  constexpr int BM = 256, WM = 4, WN = 1, TM = 4, TN = BN / 16;
  constexpr int STAGE = BN * 64;      // bf16 elements per weight stage
  constexpr int LPW = BN / 32;        // DMA instructions per wave per stage
  constexpr int AL = 2 * TM;          // activation loads per lane per stage
  static_assert(BN % 32 == 0 && NS >= 3, "tile");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NS * STAGE];

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
  const int nk = (min(K, kb + k_split) - kb) / GK;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int wm = wid, wn = 0;

  // weight rows this lane DMAs
  const bf16_t* bsrc[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int rho = (wid * LPW + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (rho & 7);
    const int gn = n0 + rho;
    const int ok = gn < N ? gn : 0;
    const int brow = (EPI == EPI_SWIGLU) ? swiglu_b_row(ok, F) : ok;
    bsrc[j] = B + (size_t)brow * ldb + c * 8;
  }
  auto issue_b = [&](int stage_k, int slot) {
    bf16_t* base = smem + slot * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[j] + stage_k), LDS_PTR(base + (wid * LPW + j) * 8 * 64),
                                       16, 0, 0);
  };
  // activation rows of this lane: m0 + 64 wid + 16 a + col, k offset quad * 8 within each 32-chunk
  const bf16_t* asrc[TM];
#pragma unroll
  for (int a = 0; a < TM; ++a) {
    const int gm = m0 + wid * 64 + a * 16 + col;
    asrc[a] = A + (size_t)(gm < Mr ? gm : 0) * lda + quad * 8;
  }
  uint4 areg[2][AL];
  auto issue_a = [&](int stage_k, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int a = 0; a < TM; ++a) areg[buf][kc * TM + a] = *(const uint4*)(asrc[a] + stage_k + kc * 32);
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = (floatx4){0.f, 0.f, 0.f, 0.f};

  // prologue: weights for stages 0..NS-2, activations for stages 0 and 1
  if (nk > 0) issue_a(kb, std::integral_constant<int, 0>());
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue_b(kb + s * GK, s);
  if (nk > 1) issue_a(kb + GK, std::integral_constant<int, 1>());

  // One iteration; the activation register buffer is a compile-time index (the loop is unrolled
  // by two) so the buffers stay in registers.
  auto step = [&](int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    // In flight, in issue order: ..., A(it+1) [issued end of it-1], B(it+NS-2) ... ; stage `it`
    // needs B(it) and A(it).  Everything issued after A(it) may stay outstanding: the weight
    // stages it+1..it+NS-2 plus A(it+1) (issued after B(it) for it >= 1).
    const int nb_after = min(NS - 2, nk - 1 - it);        // weight stages issued after B(it)
    const bool a_next = it + 1 < nk;                       // A(it+1) issued after A(it)
    if (nb_after == NS - 2 && a_next)
      wait_vmcnt_le<(NS - 2) * LPW + AL>();
    else if (a_next)
      wait_vmcnt_le<AL>();
    else
      wait_vmcnt_le<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + NS - 1 < nk) issue_b(kb + (it + NS - 1) * GK, (it + NS - 1) % NS);
    const bf16_t* st = smem + (it % NS) * STAGE;
    bf16x8_t bfr[2][TN];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int c = kc * 4 + quad;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int r = b * 16 + col;
        bfr[kc][b] = *(const bf16x8_t*)&st[r * 64 + ((c ^ (r & 7)) << 3)];
      }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const bf16x8_t af = *(const bf16x8_t*)&areg[buf][kc * TM + a];
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[kc][b], acc[a][b], 0, 0, 0);
      }
    if (it + 2 < nk) issue_a(kb + (it + 2) * GK, bufc);
  };
  for (int it = 0; it < nk; it += 2) {
    step(it, std::integral_constant<int, 0>());
    if (it + 1 < nk) step(it + 1, std::integral_constant<int, 1>());
  }
  gemm_epilogue<BM, BN, WM, WN, EPI, SPLIT>(acc, m0, n0, nt, sp, Mr, M, N, ep, wm, wn, lane, tid, (SoftStat*)smem);
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
template <int BM, int BN, int WM, int WN, int NS>
static void run_pipe(int epi, bool split, dim3 grid, const bf16_t* A, int lda, const bf16_t* B, int ldb, int M,
                     int N, int K, int k_split, int mt, int nt, int splits, const int32_t* m_dev, const GemmEpi& ep,
                     int F, hipStream_t st) {
#define GO(E, S)                                                                                             \
  k_gemm_pipe<BM, BN, WM, WN, NS, E, S><<<grid, WM * WN * 64, 0, st>>>(A, lda, B, ldb, M, N, K, k_split, mt, nt, \
                                                                       splits, m_dev, ep, F)
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

template <int BM, int BN, int NS>
static void run_wide(int epi, bool split, dim3 grid, const bf16_t* A, int lda, const bf16_t* B, int ldb, int M,
                     int N, int K, int k_split, int mt, int nt, int splits, const int32_t* m_dev, const GemmEpi& ep,
                     int F, hipStream_t st) {
#define GO(E, S)                                                                                                \
  k_gemm_wide<BM, BN, NS, E, S><<<grid, 512, 0, st>>>(A, lda, B, ldb, M, N, K, k_split, mt, nt, splits, m_dev, ep, F)
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

template <int BM, int BN, int WM, int WN, int DA, int DB>
static void run_ring2(int epi, bool split, dim3 grid, const bf16_t* A, int lda, const bf16_t* B, int ldb, int M,
                      int N, int K, int k_split, int mt, int nt, int splits, const int32_t* m_dev, const GemmEpi& ep,
                      int F, hipStream_t st) {
#define GO(E, S)                                                                                       \
  k_gemm_ring2<BM, BN, WM, WN, DA, DB, E, S><<<grid, 256, 0, st>>>(A, lda, B, ldb, M, N, K, k_split, mt, nt, \
                                                                   splits, m_dev, ep, F)
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

template <int BM, int BN, int WM, int WN, int DA, int DB>
static void run_ws(int epi, bool split, dim3 grid, const bf16_t* A, int lda, const bf16_t* B, int ldb, int M, int N,
                   int K, int k_split, int mt, int nt, int splits, const int32_t* m_dev, const GemmEpi& ep, int F,
                   hipStream_t st) {
#define GO(E, S)                                                                                             \
  k_gemm_ws<BM, BN, WM, WN, DA, DB, E, S><<<grid, WM * WN * 64, 0, st>>>(A, lda, B, ldb, M, N, K, k_split, mt, \
                                                                         nt, splits, m_dev, ep, F)
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

template <int BN, int NS>
static void run_adirect(int epi, bool split, dim3 grid, const bf16_t* A, int lda, const bf16_t* B, int ldb, int M,
                        int N, int K, int k_split, int mt, int nt, int splits, const int32_t* m_dev, const GemmEpi& ep,
                        int F, hipStream_t st) {
#define GO(E, S)                                                                                                  \
  k_gemm_adirect<BN, NS, E, S><<<grid, 256, 0, st>>>(A, lda, B, ldb, M, N, K, k_split, mt, nt, splits, m_dev, ep, \
                                                     F)
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


// Tile shapes: BM, BN and the number of waves along N.  The SwiGLU epilogue pairs gate and up
// 16-column groups inside one wave, so a single-pass SwiGLU needs an even count of column
// groups per wave (BN / WN / 16); tiles without it take SwiGLU only with split-K.
struct TileCfg {
  int bm, bn, wn;
};
static const TileCfg kTiles[] = {
    {32, 128, 4}, {64, 128, 2}, {128, 128, 2}, {256, 64, 1}, {256, 128, 1}, {128, 64, 2}, {64, 64, 2},
    {128, 256, 2},
    // pipelined (LDS ring) variants
    {128, 128, 2}, {64, 128, 2}, {32, 128, 4}, {256, 64, 1}, {64, 64, 2}, {128, 64, 2}, {256, 128, 2},
    {128, 256, 2}, {256, 96, 1}, {256, 128, 1}, {128, 96, 1},
    // activations direct to registers, weights through the LDS ring
    {256, 64, 1}, {256, 96, 1}, {256, 128, 1}, {256, 96, 1}, {256, 96, 1}, {256, 96, 1}, {256, 128, 1},
    {256, 64, 1},
    // dual ring: activation stages DA ahead, weight stages DB ahead
    {256, 96, 1}, {256, 96, 1}, {128, 96, 1}, {128, 96, 1}, {128, 128, 2}, {128, 128, 2}, {32, 128, 4},
    {64, 128, 2}, {256, 64, 1},
    // eight waves (two per SIMD), LDS ring
    {128, 192, 4}, {256, 128, 2}, {128, 128, 4}, {256, 64, 2}, {64, 192, 4}, {128, 192, 4}, {128, 128, 4},
    {128, 128, 4}, {128, 256, 4}, {64, 128, 4}, {64, 256, 4}, {128, 192, 2}, {128, 192, 2},
    // eight waves, wave-specialised loads (activation stream DA deep, weight stream DB deep)
    {128, 192, 2}, {128, 192, 2}, {128, 192, 2}, {128, 128, 4}, {128, 128, 4}, {64, 128, 4}, {256, 128, 2},
    // eight waves, deeper LDS ring
    {128, 192, 2}, {128, 128, 4}, {128, 192, 4},
    // wide tiles (many rows): eight 64-row waves, 32-deep stages, fragments prefetched (the
    // dispatcher now takes tile 64 for these shapes)
    {256, 256, 2}, {256, 256, 2}, {256, 128, 2}, {128, 256, 4}, {256, 256, 2},
    // 256 x 256 over eight 64 x 128 waves, two 64-deep stages (the whole 128-byte line of each row)
    {256, 256, 2}};
constexpr int kNumTiles = 65;

bool swiglu_single_pass_ok(int tile) { return ((kTiles[tile].bn / kTiles[tile].wn / 16) & 1) == 0; }

// Measured choices (MI355X, bf16, K = 2048..12288): rows up to 48 stream the weights with the
// 32-row pipelined tile; more rows use the eight-wave tiles (two waves per SIMD hide each other's
// LDS and barrier waits), with split-K up to 384 rows.
// Returns the tile; *splits gets the split-K factor (0 = the generic rule).
// FFN gate/up at up to 64 rows (weights streamed once, from HBM): the eight-wave 64 x 128 tile when
// its N / 128 workgroups cover three quarters of the compute units, else the four-wave 64 x 64 tile
// with twice the workgroups (weights rotated so none is cache-resident: 8B width 24576 x 4096 at
// 32 / 48 rows 40.1 / 55.0 -> 39.7 / 40.2 us, 1.7B width 12288 x 2048 at 32 / 64 rows 16.9 / 18.6 ->
// 13.8 / 14.7 us).
static int swiglu_few_rows_tile(int N) { return N >= 192 * 128 ? 45 : 12; }

int gemm_mfma_auto_tile(int epi, int M, int N, int K, int* splits) {
  *splits = 0;
  if (M <= 48) {
    if (epi == EPI_SWIGLU) {
      *splits = 1;
      return swiglu_few_rows_tile(N);
    }
    if (epi == EPI_SOFTSTAT) {
      *splits = 1;
      return 10;
    }
    // a long reduction into few outputs (1.7B FFN down: 6144 -> 2048 at 32 rows): 64 x 64 tiles
    // with split-K 8, 256 workgroups streaming the weight instead of 64 (15.7 -> 10.5 us)
    if (K > 4096 && N <= 2048) {
      *splits = 8;
      return 12;
    }
    *splits = 4;
    return N <= 4096 && K <= 4096 ? 12 : 10;
  }
  if (M <= 64 && epi == EPI_SOFTSTAT) return 9;
  if (M <= 384) {
    *splits = 1;
    // LM head: 128-row tiles up to 128 rows, then a 256 x 256 tile (one row tile, each weight
    // tile read once: 256 rows 473 -> 424 us); 257..384 rows would take two 256-row tiles, three
    // 128-row ones cost less (288 / 320 / 384 rows: 628 / 781 / 645 -> 553 / 614 / 559 us)
    if (epi == EPI_SOFTSTAT) return M <= 128 ? 47 : (M <= 256 ? 64 : 44);
    if (epi == EPI_SWIGLU) return M <= 64 ? swiglu_few_rows_tile(N) : (M <= 128 ? 18 : 56);
    // projections (QKV, O, FFN down): split-K 4 over the eight-wave tiles
    *splits = 4;
    if (M <= 128) return (M <= 64 || N <= 4096) ? 45 : 18;
    return (N > 4096 && K <= N) ? 36 : 38;
  }
  // more rows (long-context steps, prefill): single pass over the eight-wave tiles, measured at
  // 512 / 1024 / 2048 / 8192 rows on the 8B projections
  *splits = 1;
  if (epi == EPI_SOFTSTAT) return 64;  // 2048 rows: 3.24 -> 2.50 ms on the wide tile, 2.45 on tile 64
  // 256 x 256 tiles where the matrix cores bound the GEMM: every projection at >= 4096 rows
  // (8192-row prefill: gate/up 1.84 -> 1.50 ms on the wide tile), gate/up from 1536.  The
  // pipelined 256 x 256 tile (64-deep stages, two of them) does the same MFMAs in the same order
  // as the wide tile (32-deep stages, fragments read a stage ahead) and is faster at every shape
  // measured: 8192 rows gate/up 1461 -> 1369 us, QKV 397 -> 365, down 808 -> 743.
  if (M >= 4096) return 64;
  // QKV (STORE) from 1792 rows too: the long-context step's QKV (1984..2048 rows) 19.3 -> 18.5 ms
  // per step, the same tokens bit for bit
  if (M >= 1536) return epi == EPI_SWIGLU ? 64 : (epi == EPI_STORE ? (M >= 1792 ? 64 : 47) : 37);
  if (epi == EPI_SWIGLU) return M >= 768 ? 44 : 47;
  if (epi == EPI_STORE) return M >= 768 ? 47 : 38;
  return 38;
}

// The LM-head readout's column ranges.  With one row tile of a 256 x 256 tile the
// ceil(N / 256) column tiles run in rounds of one per compute unit; at N = 151936 that is 594
// tiles, 2.3 rounds, the last one a third full.  When that last round would be at most half full
// the columns of the whole rounds stay on the 256 x 256 tile and the rest run as a second launch
// on the 128 x 192 eight-wave tile, which spreads them over more workgroups (256 rows: 512 wide tiles
// 320 us + the 20864-column rest 67 us, against 437-473 us in one launch, in a probe).
void gemm_mfma_softstat_plan(int M, int N, int force_tile, SoftstatPlan* sp) {
  int s;
  const int tile = (force_tile >= 0 && force_tile < kNumTiles) ? force_tile : gemm_mfma_auto_tile(EPI_SOFTSTAT, M, N, 1, &s);
  const int bn = kTiles[tile].bn;
  sp->tile0 = tile;
  sp->cols0 = N;
  sp->tile1 = -1;
  sp->tiles0 = (N + bn - 1) / bn;
  sp->n_tiles = sp->tiles0;
  // rounds of one 512-thread 256 x 256 workgroup per compute unit (the library targets gfx950,
  // whose MI355X has 256 compute units); the rest runs on the 128 x 192 eight-wave tile
  constexpr int kCUs = 256, kRest = 47;
  if (kTiles[tile].bm >= M && kTiles[tile].bm == 256 && bn == 256) {
    const int whole = sp->tiles0 / kCUs * kCUs;
    if (whole > 0 && sp->tiles0 - whole > 0 && sp->tiles0 - whole <= kCUs / 2) {
      sp->cols0 = whole * bn;
      sp->tiles0 = whole;
      sp->tile1 = kRest;
      sp->n_tiles = whole + (N - sp->cols0 + kTiles[kRest].bn - 1) / kTiles[kRest].bn;
    }
  }
}

// Kernel and static template arguments of each tile (the names rocprofv3 reports are these with
// the epilogue and split flag appended).
struct TileName {
  const char* kernel;
  const char* args;
};
static const TileName kTileNames[kNumTiles] = {
    {"k_gemm_mfma", "32, 128, 1, 4"},
    {"k_gemm_mfma", "64, 128, 2, 2"},
    {"k_gemm_mfma", "128, 128, 2, 2"},
    {"k_gemm_mfma", "256, 64, 4, 1"},
    {"k_gemm_mfma", "256, 128, 4, 1"},
    {"k_gemm_mfma", "128, 64, 2, 2"},
    {"k_gemm_mfma", "64, 64, 2, 2"},
    {"k_gemm_mfma", "128, 256, 2, 2"},
    {"k_gemm_pipe", "128, 128, 2, 2, 4"},
    {"k_gemm_pipe", "64, 128, 2, 2, 4"},
    {"k_gemm_pipe", "32, 128, 1, 4, 6"},
    {"k_gemm_pipe", "256, 64, 4, 1, 3"},
    {"k_gemm_pipe", "64, 64, 2, 2, 6"},
    {"k_gemm_pipe", "128, 64, 2, 2, 4"},
    {"k_gemm_pipe", "256, 128, 2, 2, 3"},
    {"k_gemm_pipe", "128, 256, 2, 2, 3"},
    {"k_gemm_pipe", "256, 96, 4, 1, 3"},
    {"k_gemm_pipe", "256, 128, 4, 1, 3"},
    {"k_gemm_pipe", "128, 96, 4, 1, 4"},
    {"k_gemm_adirect", "64, 6"},
    {"k_gemm_adirect", "96, 5"},
    {"k_gemm_adirect", "128, 4"},
    {"k_gemm_adirect", "96, 3"},
    {"k_gemm_adirect", "96, 8"},
    {"k_gemm_adirect", "96, 10"},
    {"k_gemm_adirect", "128, 8"},
    {"k_gemm_adirect", "64, 12"},
    {"k_gemm_ring2", "256, 96, 4, 1, 2, 4"},
    {"k_gemm_ring2", "256, 96, 4, 1, 1, 6"},
    {"k_gemm_ring2", "128, 96, 4, 1, 2, 6"},
    {"k_gemm_ring2", "128, 96, 4, 1, 2, 8"},
    {"k_gemm_ring2", "128, 128, 2, 2, 2, 5"},
    {"k_gemm_ring2", "128, 128, 2, 2, 1, 6"},
    {"k_gemm_ring2", "32, 128, 1, 4, 2, 7"},
    {"k_gemm_ring2", "64, 128, 2, 2, 2, 7"},
    {"k_gemm_ring2", "256, 64, 4, 1, 2, 6"},
    {"k_gemm_pipe", "128, 192, 2, 4, 3"},
    {"k_gemm_pipe", "256, 128, 4, 2, 3"},
    {"k_gemm_pipe", "128, 128, 2, 4, 4"},
    {"k_gemm_pipe", "256, 64, 4, 2, 3"},
    {"k_gemm_pipe", "64, 192, 2, 4, 4"},
    {"k_gemm_pipe", "128, 192, 2, 4, 2"},
    {"k_gemm_pipe", "128, 128, 2, 4, 2"},
    {"k_gemm_pipe", "128, 128, 2, 4, 3"},
    {"k_gemm_pipe", "128, 256, 2, 4, 3"},
    {"k_gemm_pipe", "64, 128, 2, 4, 4"},
    {"k_gemm_pipe", "64, 256, 2, 4, 3"},
    {"k_gemm_pipe", "128, 192, 4, 2, 3"},
    {"k_gemm_pipe", "128, 192, 4, 2, 2"},
    {"k_gemm_ws", "128, 192, 4, 2, 2, 3"},
    {"k_gemm_ws", "128, 192, 4, 2, 1, 4"},
    {"k_gemm_ws", "128, 192, 4, 2, 2, 2"},
    {"k_gemm_ws", "128, 128, 2, 4, 2, 4"},
    {"k_gemm_ws", "128, 128, 2, 4, 2, 5"},
    {"k_gemm_ws", "64, 128, 2, 4, 2, 6"},
    {"k_gemm_ws", "256, 128, 4, 2, 2, 3"},
    {"k_gemm_pipe", "128, 192, 4, 2, 4"},
    {"k_gemm_pipe", "128, 128, 2, 4, 5"},
    {"k_gemm_pipe", "128, 192, 2, 4, 4"},
    {"k_gemm_wide", "256, 256, 4"},
    {"k_gemm_wide", "256, 256, 5"},
    {"k_gemm_wide", "256, 128, 6"},
    {"k_gemm_wide", "128, 256, 6"},
    {"k_gemm_wide", "256, 256, 3"},
    {"k_gemm_pipe", "256, 256, 4, 2, 2"},
};

// The tile and split-K the dispatcher takes for a shape (see launch_gemm_mfma).
static void gemm_choose(int epi, int M, int N, int K, size_t part_floats, int force_splits, int force_tile,
                        int* tile_out, int* splits_out) {
  int auto_splits = 0;
  int tile = (force_tile >= 0 && force_tile < kNumTiles) ? force_tile : gemm_mfma_auto_tile(epi, M, N, K,
                                                                                            &auto_splits);
  // a single-pass SwiGLU needs gate/up column pairs inside one wave: tiles without them run the
  // SwiGLU with split-K 2 (epilogue in the fixed-order reduction) or, if K cannot split, on tile 18
  const bool k_can_split = (K / GK) % 2 == 0 && (size_t)2 * M * N <= part_floats;
  if (epi == EPI_SWIGLU && !swiglu_single_pass_ok(tile) && !k_can_split) tile = 18;
  const int BM = kTiles[tile].bm, BN = kTiles[tile].bn;
  const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  int splits = 1;
  if (epi != EPI_SOFTSTAT) {
    if (force_splits > 0) {
      splits = force_splits;
    } else if (auto_splits > 0 && force_tile < 0) {
      splits = auto_splits;
    } else {
      while (mt * nt * splits < 512 && (K / GK) % (splits * 2) == 0 && K / (splits * 2) >= 512 &&
             (size_t)(splits * 2) * M * N <= part_floats)
        splits *= 2;
    }
    if ((size_t)splits * M * N > part_floats || (K / GK) % splits != 0) splits = 1;
    if (epi == EPI_SWIGLU && splits == 1 && !swiglu_single_pass_ok(tile)) splits = 2;  // k_can_split holds here
  }
  *tile_out = tile;
  *splits_out = splits;
}

// Chooses the tile and split-K, then launches.  For SWIGLU, N = 2F (interleaved gate/up columns)
// and the output has F columns.  part/part_floats: split-K scratch.  force_tile / force_splits
// (>= 0 / > 0) override the choice.
int launch_gemm_mfma(int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                     const int32_t* m_dev, const GemmEpi& ep, int F, float* part, size_t part_floats,
                     int force_splits, hipStream_t st, int force_tile, bool defer_reduce) {
  if (M <= 0 || N <= 0) return 1;
  int tile, splits;
  gemm_choose(epi, M, N, K, part_floats, force_splits, force_tile, &tile, &splits);
  const int BM = kTiles[tile].bm, BN = kTiles[tile].bn;
  const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
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
#define T(BM_, BN_, WM_, WN_) \
  run_tile<BM_, BN_, WM_, WN_>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st)
  switch (tile) {
    case 0: T(32, 128, 1, 4); break;
    case 1: T(64, 128, 2, 2); break;
    case 2: T(128, 128, 2, 2); break;
    case 3: T(256, 64, 4, 1); break;
    case 4: T(256, 128, 4, 1); break;
    case 5: T(128, 64, 2, 2); break;
    case 6: T(64, 64, 2, 2); break;
    case 7: T(128, 256, 2, 2); break;
#define P(BM_, BN_, WM_, WN_, NS_) \
  run_pipe<BM_, BN_, WM_, WN_, NS_>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st)
    case 8: P(128, 128, 2, 2, 4); break;
    case 9: P(64, 128, 2, 2, 4); break;
    case 10: P(32, 128, 1, 4, 6); break;
    case 11: P(256, 64, 4, 1, 3); break;
    case 12: P(64, 64, 2, 2, 6); break;
    case 13: P(128, 64, 2, 2, 4); break;
    case 14: P(256, 128, 2, 2, 3); break;
    case 15: P(128, 256, 2, 2, 3); break;
    case 16: P(256, 96, 4, 1, 3); break;
    case 17: P(256, 128, 4, 1, 3); break;
    case 18: P(128, 96, 4, 1, 4); break;
#undef P
#define D(BN_, NS_) \
  run_adirect<BN_, NS_>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st)
    case 19: D(64, 6); break;
    case 20: D(96, 5); break;
    case 21: D(128, 4); break;
    case 23: D(96, 8); break;
    case 24: D(96, 10); break;
    case 25: D(128, 8); break;
    case 26: D(64, 12); break;
    default: D(96, 3); break;
#undef D
#define R(BM_, BN_, WM_, WN_, DA_, DB_)                                                                        \
  run_ring2<BM_, BN_, WM_, WN_, DA_, DB_>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, \
                                         e, F, st)
    case 27: R(256, 96, 4, 1, 2, 4); break;
    case 28: R(256, 96, 4, 1, 1, 6); break;
    case 29: R(128, 96, 4, 1, 2, 6); break;
    case 30: R(128, 96, 4, 1, 2, 8); break;
    case 31: R(128, 128, 2, 2, 2, 5); break;
    case 32: R(128, 128, 2, 2, 1, 6); break;
    case 33: R(32, 128, 1, 4, 2, 7); break;
    case 34: R(64, 128, 2, 2, 2, 7); break;
    case 35: R(256, 64, 4, 1, 2, 6); break;
#undef R
#define P8(BM_, BN_, WM_, WN_, NS_) \
  run_pipe<BM_, BN_, WM_, WN_, NS_>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st)
    case 36: P8(128, 192, 2, 4, 3); break;
    case 37: P8(256, 128, 4, 2, 3); break;
    case 38: P8(128, 128, 2, 4, 4); break;
    case 39: P8(256, 64, 4, 2, 3); break;
    case 40: P8(64, 192, 2, 4, 4); break;
    case 41: P8(128, 192, 2, 4, 2); break;
    case 42: P8(128, 128, 2, 4, 2); break;
    case 43: P8(128, 128, 2, 4, 3); break;
    case 44: P8(128, 256, 2, 4, 3); break;
    case 45: P8(64, 128, 2, 4, 4); break;
    case 46: P8(64, 256, 2, 4, 3); break;
    case 47: P8(128, 192, 4, 2, 3); break;
    case 48: P8(128, 192, 4, 2, 2); break;
#define W(BM_, BN_, WM_, WN_, DA_, DB_) \
  run_ws<BM_, BN_, WM_, WN_, DA_, DB_>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st)
    case 49: W(128, 192, 4, 2, 2, 3); break;
    case 50: W(128, 192, 4, 2, 1, 4); break;
    case 51: W(128, 192, 4, 2, 2, 2); break;
    case 52: W(128, 128, 2, 4, 2, 4); break;
    case 53: W(128, 128, 2, 4, 2, 5); break;
    case 54: W(64, 128, 2, 4, 2, 6); break;
    case 55: W(256, 128, 4, 2, 2, 3); break;
#undef W
    // four and five stages: the full 160 KB of LDS
    case 56: P8(128, 192, 4, 2, 4); break;
    case 57: P8(128, 128, 2, 4, 5); break;
    case 58: P8(128, 192, 2, 4, 4); break;
#undef P8
#define WD(BM_, BN_, NS_) \
  run_wide<BM_, BN_, NS_>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st)
    case 59: WD(256, 256, 4); break;
    case 60: WD(256, 256, 5); break;
    case 61: WD(256, 128, 6); break;
    case 62: WD(128, 256, 6); break;
    case 63: WD(256, 256, 3); break;
#undef WD
    case 64: run_pipe<256, 256, 4, 2, 2>(epi, split, grid, a, lda, b, ldb, M, N, K, k_split, mt, nt, splits, m_dev, e, F, st); break;

  }
#undef T
  if (split && !(defer_reduce && epi != EPI_SWIGLU)) {
    const int NO = epi == EPI_SWIGLU ? N / 2 : N;
    const size_t n = (size_t)M * NO;
    const unsigned g = (unsigned)((n + 255) / 256);
    if (epi == EPI_SWIGLU)
      k_splitk_reduce<EPI_SWIGLU><<<g, 256, 0, st>>>(part, splits, M, N, m_dev, ep);
    else if (epi == EPI_RESID)
      k_splitk_reduce<EPI_RESID><<<g, 256, 0, st>>>(part, splits, M, N, m_dev, ep);
    else
      k_splitk_reduce<EPI_STORE><<<g, 256, 0, st>>>(part, splits, M, N, m_dev, ep);
    return 1;
  }
  return splits;
}

}  // namespace alodlm

#include "../../include/alodlm_diag.h"

extern "C" int alodlm_diag_gemm(int32_t epi, int32_t M, int32_t N, int32_t K, const void* A, const void* B, float* C,
                                void* act, float* scratch, size_t scratch_floats, int32_t force_splits,
                                int32_t force_generic, int32_t force_tile, void* hip_stream) {
  using namespace alodlm;
  if (M <= 0 || N <= 0 || K <= 0 || !A || !B) return -1;
  if (epi == EPI_SOFTSTAT) {
    if (!C || !act || !scratch || force_generic || !gemm_mfma_supported(K, K, K)) return -1;
    int sp;
    const int tile = (force_tile >= 0 && force_tile < kNumTiles) ? force_tile : gemm_mfma_auto_tile(epi, M, N, K, &sp);
    const int n_tiles = (N + kTiles[tile].bn - 1) / kTiles[tile].bn;
    if ((size_t)4 * M * n_tiles > scratch_floats) return -1;
    hipStream_t st = (hipStream_t)hip_stream;
    float* H = C;                 // first M floats, then the M log-sum-exps
    float* lse = C + M;
    GemmEpi ep;
    ep.part = (SoftStat*)scratch;
    ep.n_tiles = n_tiles;
    launch_gemm_mfma(epi, A, K, B, K, M, N, K, nullptr, ep, 0, nullptr, 0, 1, st, tile, false);
    launch_softstat_combine((const SoftStat*)scratch, M, n_tiles, nullptr, H, lse, (int32_t*)act, nullptr, nullptr,
                            st);
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
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
                     force_splits, st, force_tile, false);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int alodlm_diag_gemm_choice(int32_t epi, int32_t M, int32_t N, int32_t K, size_t scratch_floats,
                                       int32_t* tile, int32_t* splits, char* name, size_t name_len) {
  using namespace alodlm;
  if (M <= 0 || N <= 0 || K <= 0 || !gemm_mfma_supported(K, K, K) || epi < 0 || epi > 3) return -1;
  int t, sp;
  gemm_choose(epi, M, N, K, scratch_floats, 0, -1, &t, &sp);
  if (tile) *tile = t;
  if (splits) *splits = sp;
  if (epi == EPI_SOFTSTAT) {  // the readout's column ranges (one or two launches)
    SoftstatPlan rp;
    gemm_mfma_softstat_plan(M, N, -1, &rp);
    if (tile) *tile = rp.tile0;
    if (name && name_len) {
      if (rp.tile1 < 0)
        snprintf(name, name_len, "%s<%s, %d, false>", kTileNames[rp.tile0].kernel, kTileNames[rp.tile0].args, epi);
      else
        snprintf(name, name_len, "%s<%s, %d, false> (columns 0..%d) + %s<%s, %d, false> (columns %d..%d)",
                 kTileNames[rp.tile0].kernel, kTileNames[rp.tile0].args, epi, rp.cols0 - 1,
                 kTileNames[rp.tile1].kernel, kTileNames[rp.tile1].args, epi, rp.cols0, N - 1);
    }
    return 0;
  }
  if (name && name_len) {
    // the instantiation the dispatcher launches: split-K STORE / RESID run the plain store epilogue
    const int e = sp > 1 ? (epi == EPI_SWIGLU ? EPI_SWIGLU : EPI_STORE) : epi;
    snprintf(name, name_len, "%s<%s, %d, %s>", kTileNames[t].kernel, kTileNames[t].args, e, sp > 1 ? "true" : "false");
  }
  return 0;
}

extern "C" int alodlm_diag_readout_sample(int32_t M, int32_t N, int32_t K, const void* A, const void* B,
                                          const int32_t* row_key, uint64_t seed, uint32_t c2, uint32_t c3,
                                          int32_t* tok, float* scratch, size_t scratch_floats,
                                          int32_t force_generic, int32_t force_tile, void* hip_stream) {
  using namespace alodlm;
  if (M <= 0 || N <= 0 || K <= 0 || !A || !B || !row_key || !tok || !scratch) return -1;
  const bool mfma = !force_generic && gemm_mfma_supported(K, K, K);
  int sp;
  const int tile = !mfma ? -1
                         : ((force_tile >= 0 && force_tile < kNumTiles) ? force_tile
                                                                        : gemm_mfma_auto_tile(EPI_SOFTSTAT, M, N, K, &sp));
  const int bn = mfma ? kTiles[tile].bn : 64;
  const int n_tiles = (N + bn - 1) / bn;
  const size_t need = (size_t)6 * M * n_tiles + (size_t)3 * M;
  if (need > scratch_floats) return -1;
  hipStream_t st = (hipStream_t)hip_stream;
  GemmEpi ep;
  ep.part = (SoftStat*)scratch;
  ep.n_tiles = n_tiles;
  ep.smp.part = (GStat*)(scratch + (size_t)4 * M * n_tiles);
  ep.smp.row_key = row_key;
  ep.smp.k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  ep.smp.k1 = (uint32_t)(seed >> 32);
  ep.smp.c2 = c2;
  ep.smp.c3 = c3;
  if (mfma)
    launch_gemm_mfma(EPI_SOFTSTAT, A, K, B, K, M, N, K, nullptr, ep, 0, nullptr, 0, 1, st, tile, false);
  else
    launch_gemm_generic(DT_BF16, EPI_SOFTSTAT, A, K, B, K, M, N, K, nullptr, ep, st);
  float* H = scratch + (size_t)6 * M * n_tiles;
  launch_softstat_combine((const SoftStat*)scratch, M, n_tiles, nullptr, H, H + M, (int32_t*)(H + 2 * M), ep.smp.part,
                          tok, st);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
