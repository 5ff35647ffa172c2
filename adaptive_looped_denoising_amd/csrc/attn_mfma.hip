// Block attention over the depth-aware prefix cache on the gfx950 matrix cores (bf16).
//
// One workgroup (4 waves) takes one (sequence slot, kv head) pair, a block of QB query rows of
// that pair -- the G = Hq/Hkv query heads sharing the kv head are packed as rows
// (position i, head g) -> i*G + g -- and one split of its key range.  Keys are the prefix keys
// (Core layers read position j at depth min(loop, avail[j]), gathered row by row from the depth
// planes) followed by the block's own keys.  Per tile of 64 keys:
//   K tile -> LDS (key-major), V tile -> LDS transposed ([hd][key]);
//   S^T = K Q^T on the matrix cores (Q held in registers as the B operand), so every lane ends
//   up with 16 scores of one query column -- the online softmax needs no LDS round trip and the
//   probabilities are already laid out as the B operand of O^T += V^T P^T;
//   O^T accumulates in registers (fp32), rescaled by the running-max correction.
// With several key splits, partial (O, max, sum) go to a scratch buffer and k_attn_merge
// combines them in a fixed order.
#include "common.h"
#include "launch.h"

namespace alodlm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int AKT = 64;  // keys per tile

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)from_f<bf16_t>(lo) | ((uint32_t)from_f<bf16_t>(hi) << 16);
}

// Address of key j (0-based over prefix keys then own keys) of sequence slot t / cache sequence b.
// Core layers take the depth plane of prefix key j from sdep[j - dep_base] (staged in LDS).
__device__ __forceinline__ const bf16_t* akv_row(const AttnParams& p, const void* cbase, const void* sbase, int j,
                                                 int b, int t, int kvh, const uint8_t* sdep, int dep_base) {
  if (j < p.n_cache) {
    size_t off = (size_t)b * p.c_sSeq + (size_t)kvh * p.c_sHead + (size_t)j * p.c_sPos;
    if (p.core) off += (size_t)sdep[j - dep_base] * p.c_plane;
    return (const bf16_t*)cbase + off;
  }
  const int jj = j - p.n_cache;
  return (const bf16_t*)sbase + (size_t)(t + p.s_seq0) * p.s_sSeq + (size_t)kvh * p.s_sHead + (size_t)jj * p.s_sPos;
}

template <int HD, int QW>
__global__ __launch_bounds__(256) void k_attn_mfma(AttnParams p, int n_pairs, int n_qblocks, int n_splits,
                                                   int keys_per_split) {
  constexpr int QB = 4 * QW;
  constexpr int NQ = QW / 16;
  constexpr int NH = HD / 16;
  constexpr int NC = HD / 32;
  constexpr int CPR = HD / 8;          // 16-byte chunks per key row
  constexpr int KLD = HD + 8;          // K tile pitch (elements)
  constexpr int VLD = AKT + 4;         // V^T tile pitch (keys)
  constexpr int KROWS = 256 / CPR;     // key rows loaded per pass
  constexpr int DEPC = 4096;            // depth-plane indices staged per chunk of prefix keys
  __shared__ __attribute__((aligned(16))) bf16_t sK[AKT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[HD * VLD];
  __shared__ uint8_t sdep[DEPC];

  const int total = n_pairs * n_qblocks * n_splits;
  const int per = (gridDim.x + 7) >> 3;
  const int T = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (T >= total) return;
  const int qb = T % n_qblocks;
  const int sp = (T / n_qblocks) % n_splits;
  const int pair = T / (n_qblocks * n_splits);
  const int t = pair / p.Hkv, kvh = pair % p.Hkv;
  const int b = p.seq_map ? p.seq_map[t] : t;
  const int G = p.Hq / p.Hkv;
  const int rows_q = G * p.rows_per_seq;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;

  // key range of this block
  const int n_keys = p.n_cache + p.n_self;
  int kbeg = sp * keys_per_split;
  int kend = min(n_keys, kbeg + keys_per_split);
  if (p.causal) {  // last position of the block's queries bounds the keys it can see
    const int last_row = min(rows_q, (qb + 1) * QB) - 1;
    kend = min(kend, p.n_cache + last_row / G + 1);
  }

  // Q fragments (B operand): query row rho = qb*QB + wid*QW + nq*16 + col, hd chunk c
  bf16x8_t qf[NQ][NC];
  int qpos[NQ];
  bool qok[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const int rho = qb * QB + wid * QW + nq * 16 + col;
    qok[nq] = rho < rows_q;
    const int i = qok[nq] ? rho / G : 0, g = qok[nq] ? rho % G : 0;
    qpos[nq] = i;
    const bf16_t* qp = (const bf16_t*)p.q + ((size_t)(t * p.rows_per_seq + i) * p.Hq + kvh * G + g) * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 v = qok[nq] ? *(const uint4*)(qp + c * 32 + quad * 8) : make_uint4(0, 0, 0, 0);
      qf[nq][c] = *(bf16x8_t*)&v;
    }
  }

  floatx4 o[NH][NQ];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) o[h][nq] = (floatx4){0.f, 0.f, 0.f, 0.f};
  float mrun[NQ], lrun[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    mrun[nq] = -INFINITY;
    lrun[nq] = 0.f;
  }

  // K/V tile loads are register double-buffered: the next tile's rows are in flight while the
  // matrix cores work on the current one.
  constexpr int KP = AKT / KROWS;  // K row passes per thread
  uint4 kreg[KP], vreg[4];
  const bool vthread = tid < 16 * CPR;
  int dep_base = kbeg;
  auto gload = [&](int k0) {
#pragma unroll
    for (int pass = 0; pass < KP; ++pass) {
      const int j = k0 + pass * KROWS + tid / CPR;
      kreg[pass] = j < kend ? *(const uint4*)(akv_row(p, p.ck, p.sk, j, b, t, kvh, sdep, dep_base) + (tid % CPR) * 8)
                            : make_uint4(0, 0, 0, 0);
    }
    if (vthread) {
      const int kq = tid / CPR, c = tid % CPR;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = k0 + kq * 4 + u;
        vreg[u] = j < kend ? *(const uint4*)(akv_row(p, p.cv, p.sv, j, b, t, kvh, sdep, dep_base) + c * 8)
                           : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int pass = 0; pass < KP; ++pass) {
      const int r = pass * KROWS + tid / CPR, c = tid % CPR;
      *(uint4*)&sK[r * KLD + c * 8] = kreg[pass];
    }
    if (vthread) {  // transpose: 4 consecutive keys x 8 hd values -> 8 rows of V^T
      const int kq = tid / CPR, c = tid % CPR;
      const bf16_t* e0 = (const bf16_t*)&vreg[0];
      const bf16_t* e1 = (const bf16_t*)&vreg[1];
      const bf16_t* e2 = (const bf16_t*)&vreg[2];
      const bf16_t* e3 = (const bf16_t*)&vreg[3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 w;
        w.x = (uint32_t)e0[e] | ((uint32_t)e1[e] << 16);
        w.y = (uint32_t)e2[e] | ((uint32_t)e3[e] << 16);
        *(uint2*)&sV[(c * 8 + e) * VLD + kq * 4] = w;
      }
    }
  };
  // depth plane min(loop, avail[j]) - 1 of the prefix keys [kstart, kstart + DEPC) of this range
  auto load_dep = [&](int kstart) {
    const int lim = min(min(kend, p.n_cache), kstart + DEPC);
    for (int j = kstart + tid; j < lim; j += 256)
      sdep[j - kstart] = (uint8_t)(max(1, min(p.loop, (int)p.avail[(size_t)b * p.av_stride + j])) - 1);
  };
  if (p.core) {
    load_dep(kbeg);
    __syncthreads();
  }
  if (kbeg < kend) gload(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += AKT) {
    __syncthreads();
    sstore();
    __syncthreads();
    const int kn = k0 + AKT;
    if (kn < kend) {
      if (p.core && (kn - dep_base) >= DEPC) {  // next tile starts a new chunk of staged depths
        dep_base = kn;
        load_dep(kn);
        __syncthreads();
      }
      gload(kn);
    }

    // S^T = K Q^T : 4 key subtiles x NQ query subtiles
    floatx4 s[4][NQ];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) s[ks][nq] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)&sK[(ks * 16 + col) * KLD + c * 32 + quad * 8];
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) s[ks][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[nq][c], s[ks][nq], 0, 0, 0);
      }
    }

    // online softmax per query column; probabilities packed as the B operand of the PV product
    bf16x8_t pb[2][NQ];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      float mx = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = k0 + ks * 16 + quad * 4 + v;
          bool ok = j < kend && qok[nq];
          if (p.causal) ok = ok && (j < p.n_cache || j - p.n_cache <= qpos[nq]);
          const float sc = ok ? s[ks][nq][v] * p.scale : -INFINITY;
          s[ks][nq][v] = sc;
          mx = fmaxf(mx, sc);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrun[nq], mx);
      const float corr = mnew == -INFINITY ? 1.f : __expf(mrun[nq] - mnew);
      float sum = 0.f;
      float pv[4][4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float e = mnew == -INFINITY ? 0.f : __expf(s[ks][nq][v] - mnew);
          pv[ks][v] = e;
          sum += e;
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      lrun[nq] = lrun[nq] * corr + sum;
      mrun[nq] = mnew;
#pragma unroll
      for (int h = 0; h < NH; ++h) o[h][nq] *= corr;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        uint4 w;
        w.x = pack_bf16x2(pv[2 * c2][0], pv[2 * c2][1]);
        w.y = pack_bf16x2(pv[2 * c2][2], pv[2 * c2][3]);
        w.z = pack_bf16x2(pv[2 * c2 + 1][0], pv[2 * c2 + 1][1]);
        w.w = pack_bf16x2(pv[2 * c2 + 1][2], pv[2 * c2 + 1][3]);
        pb[c2][nq] = *(bf16x8_t*)&w;
      }
    }

    // O^T += V^T P^T ; lane's 8 k-slots are keys 32c2 + 4quad + {0..3} and 32c2 + 16 + 4quad + {0..3}
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16_t* vr = &sV[(h * 16 + col) * VLD + c2 * 32 + quad * 4];
        uint4 w;
        const uint2 lo = *(const uint2*)vr;
        const uint2 hi = *(const uint2*)(vr + 16);
        w.x = lo.x;
        w.y = lo.y;
        w.z = hi.x;
        w.w = hi.y;
        const bf16x8_t a = *(bf16x8_t*)&w;
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) o[h][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[c2][nq], o[h][nq], 0, 0, 0);
      }
    }
  }

  // write: lane holds query column col of subtile nq, hd rows h*16 + 4*quad + v
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    if (!qok[nq]) continue;
    const int rho = qb * QB + wid * QW + nq * 16 + col;
    const int i = rho / G, g = rho % G;
    if (n_splits == 1) {
      const float inv = lrun[nq] > 0.f ? 1.0f / lrun[nq] : 0.f;
      bf16_t* out = (bf16_t*)p.out + (size_t)(t * p.rows_per_seq + i) * p.Hq * HD + (size_t)(kvh * G + g) * HD;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        uint2 w;
        w.x = pack_bf16x2(o[h][nq][0] * inv, o[h][nq][1] * inv);
        w.y = pack_bf16x2(o[h][nq][2] * inv, o[h][nq][3] * inv);
        *(uint2*)&out[h * 16 + quad * 4] = w;
      }
    } else {
      float* part = p.part + (((size_t)pair * rows_q + rho) * n_splits + sp) * (HD + 2);
#pragma unroll
      for (int h = 0; h < NH; ++h) *(float4*)&part[h * 16 + quad * 4] = make_float4(o[h][nq][0], o[h][nq][1], o[h][nq][2], o[h][nq][3]);
      if (quad == 0) {
        part[HD] = mrun[nq];
        part[HD + 1] = lrun[nq];
      }
    }
  }
}

// Combine the key splits of each (pair, query row) in a fixed order.
template <int HD>
__global__ __launch_bounds__(256) void k_attn_merge(AttnParams p, int n_pairs, int n_splits) {
  const int G = p.Hq / p.Hkv;
  const int rows_q = G * p.rows_per_seq;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= n_pairs * rows_q) return;
  const int pair = w / rows_q, rho = w % rows_q;
  const int t = pair / p.Hkv, kvh = pair % p.Hkv;
  const int i = rho / G, g = rho % G;
  const float* part = p.part + ((size_t)pair * rows_q + rho) * n_splits * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part[s * (HD + 2) + HD]);
  float L = 0.f, acc[(HD + 63) / 64];
#pragma unroll
  for (int u = 0; u < (HD + 63) / 64; ++u) acc[u] = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const float* ps = part + s * (HD + 2);
    const float ms = ps[HD];
    const float f = ms == -INFINITY ? 0.f : __expf(ms - M);
    L += f * ps[HD + 1];
#pragma unroll
    for (int u = 0; u < (HD + 63) / 64; ++u) {
      const int e = lane + 64 * u;
      if (e < HD) acc[u] += f * ps[e];
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  bf16_t* out = (bf16_t*)p.out + (size_t)(t * p.rows_per_seq + i) * p.Hq * HD + (size_t)(kvh * G + g) * HD;
#pragma unroll
  for (int u = 0; u < (HD + 63) / 64; ++u) {
    const int e = lane + 64 * u;
    if (e < HD) out[e] = from_f<bf16_t>(acc[u] * inv);
  }
}

template <int HD, int QW>
static void run_attn(const AttnParams& p, int n_pairs, int n_qblocks, int n_splits, int kps, hipStream_t st) {
  const int total = n_pairs * n_qblocks * n_splits;
  const int grid = ((total + 7) / 8) * 8;
  k_attn_mfma<HD, QW><<<grid, 256, 0, st>>>(p, n_pairs, n_qblocks, n_splits, kps);
  if (n_splits > 1) {
    const int rows_q = (p.Hq / p.Hkv) * p.rows_per_seq;
    const int waves = n_pairs * rows_q;
    k_attn_merge<HD><<<(waves + 3) / 4, 256, 0, st>>>(p, n_pairs, n_splits);
  }
}

bool attn_mfma_supported(int hd) { return hd == 32 || hd == 64 || hd == 128; }

// p.n_rows / rows_per_seq = sequence slots; p.part must hold n_pairs * rows_q * max_splits * (hd + 2)
// floats when max_splits > 1.
void launch_attn_mfma(const AttnParams& p, int max_splits, hipStream_t st, int force_splits, int force_qw) {
  if (p.n_rows <= 0) return;
  const int n_seq = p.n_rows / p.rows_per_seq;
  const int n_pairs = n_seq * p.Hkv;
  const int rows_q = (p.Hq / p.Hkv) * p.rows_per_seq;
  // 16 query rows per wave measured faster than 32 at 128 query rows per pair (more blocks in
  // flight per key range); 32 only where one pair has more than 256 query rows
  const int QW = (force_qw == 16 || force_qw == 32) ? force_qw : (rows_q <= 256 ? 16 : 32);
  const int QB = 4 * QW;
  const int n_qblocks = (rows_q + QB - 1) / QB;
  const int n_keys = p.n_cache + p.n_self;
  const int n_tiles = (n_keys + AKT - 1) / AKT;
  int splits = 1;
  if (!p.causal && p.part) {
    // about three resident blocks per compute unit, and at least 3 key tiles per split
    const int want = (768 + n_pairs * n_qblocks - 1) / (n_pairs * n_qblocks);
    splits = min(min(want, max(1, (n_tiles + 2) / 3)), max_splits);
    if (force_splits > 0) splits = min(force_splits, max_splits);
    if (splits < 1) splits = 1;
  }
  const int kps = ((n_tiles + splits - 1) / splits) * AKT;
  splits = (n_keys + kps - 1) / kps;
  if (splits < 1) splits = 1;
#define GO(H, Q) run_attn<H, Q>(p, n_pairs, n_qblocks, splits, kps, st)
  if (p.hd == 128) {
    if (QW == 16) GO(128, 16); else GO(128, 32);
  } else if (p.hd == 64) {
    if (QW == 16) GO(64, 16); else GO(64, 32);
  } else {
    if (QW == 16) GO(32, 16); else GO(32, 32);
  }
#undef GO
}

}  // namespace alodlm
