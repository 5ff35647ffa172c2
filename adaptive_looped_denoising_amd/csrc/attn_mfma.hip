// Block attention over the depth-aware prefix cache on the gfx950 matrix cores (bf16).
//
// One workgroup (NW = 4 or 8 waves) takes one (sequence slot, kv head) pair, a block of
// QB = NW * QW query rows of that pair -- the G = Hq/Hkv query heads sharing the kv head are packed as rows
// (position i, head g) -> i*G + g -- and one split of its key tiles.  Key tiles hold 64 keys of
// one segment: the prefix keys (the cache slot of the loop's depth plane; the planes are
// materialised at prefill so that plane s already holds every position at depth
// min(s, available depth)), then the block's own keys.
//
// Both operand tiles stream straight from memory into an NS-stage LDS ring with direct
// global->LDS loads, no register staging and no transposition:
//   K tile [64 keys][HD] (hd-contiguous rows), 16-byte chunks XOR-swizzled by row (kswz);
//   V^T tile [HD][64 keys] -- the cache stores V transposed (positions contiguous), which is
//   the operand layout of the P.V product -- chunks swizzled by (row / 2).
// S^T = K Q^T on the matrix cores (Q in registers as the B operand), so every lane holds 16
// scores of one query column: the online softmax needs no LDS round trip and the
// probabilities are already laid out as the B operand of O^T += V^T P^T.  The rows of each
// 16-key S product are a permutation of the tile's keys chosen so that the 8 probabilities a
// lane feeds one P.V product are 8 consecutive keys: each V^T fragment is then one 16-byte
// chunk of a row.
// With several key splits, partial (O, max, sum) go to a scratch buffer and k_attn_merge
// combines them in a fixed order.
// KH = 2 (key halves): two waves share each 16-row query sub-block, one taking keys 0..31 and
// the other keys 32..63 of every tile (S subtiles 0-1 / 2-3, which are exactly the keys of P.V
// products 0 / 1), each with its own online softmax; at the end the second wave hands (max, sum,
// O) to the first through LDS.  Four waves then cover 32 query rows and stream every key tile of
// the pair, so the four 32-row blocks of a 128-row pair need no key split and no merge launch:
// they run side by side on one XCD and read each K/V tile from its L2.
// F8: keys and values are stored in FP8 E4M3 (half the bytes).  The fp8 tiles stream into the
// LDS ring unswizzled; once a stage has landed, the workgroup converts it (exactly: every E4M3
// value is a bf16 value) into one bf16 working tile in the layout above, and the matrix-core
// code is unchanged.
#include "common.h"
#include "launch.h"

namespace alodlm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int AKT = 64;  // keys per tile

// Key of row i (0..15) of the ks-th 16-row S product: subtiles 2c and 2c+1 interleave the keys
// of 32-key group c in blocks of four, so lane quad q (rows 4q .. 4q+3) of the pair holds keys
// 32c + 8q .. 32c + 8q + 7.
__device__ __forceinline__ int s_key(int ks, int i) { return (ks >> 1) * 32 + (i >> 2) * 8 + (ks & 1) * 4 + (i & 3); }

// K-tile chunk swizzle: the 16 key rows one S fragment read touches (b + {0..3, 8..11, 16..19,
// 24..27}) fall in distinct LDS banks.
template <int HD>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (HD == 128) return (r & 3) | (((r >> 3) & 3) << 2);
  else if constexpr (HD == 64) return ((r >> 1) & 1) | (((r >> 3) & 3) << 1);
  else return (r >> 3) & 3;
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two floats as two bf16 (round to nearest even) in one 32-bit word, lo in the low half: one
// packed conversion instruction on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const float2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

// Two E4M3 bytes of w (the low half when HI is false, else the high half) as two bf16 (exact:
// bf16 keeps 7 fraction bits).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  const float2v f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xFFFF0000u);
}

// 16 E4M3 values -> two groups of 8 bf16 (elements 0..7, 8..15).
__device__ __forceinline__ void fp8x16_to_bf16(const uint4 in, uint4& lo, uint4& hi) {
  lo.x = fp8x2_to_bf16x2<false>(in.x);
  lo.y = fp8x2_to_bf16x2<true>(in.x);
  lo.z = fp8x2_to_bf16x2<false>(in.y);
  lo.w = fp8x2_to_bf16x2<true>(in.y);
  hi.x = fp8x2_to_bf16x2<false>(in.z);
  hi.y = fp8x2_to_bf16x2<true>(in.z);
  hi.z = fp8x2_to_bf16x2<false>(in.w);
  hi.w = fp8x2_to_bf16x2<true>(in.w);
}

// NW waves per workgroup (4, or 8 for HD >= 64: two waves per SIMD sharing one K/V stream).
template <int HD, int QW, int NS, int NW, bool F8, int KH>
__global__ __launch_bounds__(NW * 64) void k_attn_mfma(AttnParams p, int n_pairs, int n_qblocks, int n_splits,
                                                       int tiles_per_split) {
  static_assert(KH == 1 || (KH == 2 && !F8), "key halves: bf16 K/V only");
  constexpr int QB = NW / KH * QW;
  constexpr int KS = 4 / KH;             // 16-key S subtiles of a tile per wave
  constexpr int C2 = 2 / KH;             // 32-key P.V products of a tile per wave
  constexpr int NQ = QW / 16;
  constexpr int NH = HD / 16;
  constexpr int NC = HD / 32;
  constexpr int CK = HD / 8;             // 16-byte chunks per K row
  constexpr int KST = AKT * HD;          // K elements per stage
  constexpr int STAGE = 2 * AKT * HD;    // K then V^T
  constexpr int KL = HD * 8 / (64 * NW) / (F8 ? 2 : 1); // K load instructions per wave per stage (1 KB each)
  constexpr int VL = KL;                                 // V^T load instructions per wave per stage
  constexpr int LPW = KL + VL;
  constexpr int RPI = 1024 / (HD * 2);   // K rows per load instruction
  constexpr int CK8 = HD / 16;           // fp8: 16-byte chunks per K row
  constexpr int STAGE8 = 2 * AKT * HD;   // fp8: bytes per ring stage (K then V^T)
  static_assert(KL >= 1 && KL * NW * 64 * (F8 ? 2 : 1) == HD * 8, "tile loads must split evenly over the waves");
  static_assert(NS >= 2 && (NS - 2) * LPW < 64, "ring depth");
  // bf16: NS stages; fp8: NS fp8 stages, then the bf16 working tile
  constexpr int SMEM = F8 ? NS * STAGE8 / 2 + STAGE : NS * STAGE;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[SMEM];
  char* const ring8 = (char*)smem;
  bf16_t* const work = smem + (F8 ? NS * STAGE8 / 2 : 0);

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
  const int wq = wid / KH, kh = wid % KH;  // query sub-block, key half

  // tile range of this block: prefix tiles 0 .. TP-1, then own-key tiles TP .. TP+TS-1
  const int TP = (p.n_cache + AKT - 1) / AKT;
  int TE = TP + (p.n_self + AKT - 1) / AKT;
  if (p.causal) {  // the block's last query position bounds the own keys it can see
    const int last_row = min(rows_q, (qb + 1) * QB) - 1;
    TE = min(TE, TP + (last_row / G + p.causal_off) / AKT + 1);
  }
  const int tb = sp * tiles_per_split;
  const int te = min(TE, tb + tiles_per_split);

  // Q fragments (B operand): query row rho = qb*QB + wid*QW + nq*16 + col, hd chunk c
  bf16x8_t qf[NQ][NC];
  int qpos[NQ];
  bool qok[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const int rho = qb * QB + wq * QW + nq * 16 + col;
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

  const float scale2 = p.scale * 1.44269504088896341f;  // softmax scale times log2(e)

  // segment bases of this (sequence, kv head)
  const bf16_t* kpre = (const bf16_t*)p.ck + (size_t)b * p.c_kSeq + (size_t)kvh * p.c_kHead;
  const bf16_t* vpre = (const bf16_t*)p.cv + (size_t)b * p.c_vSeq + (size_t)kvh * p.c_vHead;
  const bf16_t* kslf = (const bf16_t*)p.sk + (size_t)(t + p.s_seq0) * p.s_kSeq + (size_t)kvh * p.s_kHead;
  const bf16_t* vslf = (const bf16_t*)p.sv + (size_t)(t + p.s_seq0) * p.s_vSeq + (size_t)kvh * p.s_vHead;
  // the same bases for one-byte (fp8) elements
  const char* kpre8 = (const char*)p.ck + (size_t)b * p.c_kSeq + (size_t)kvh * p.c_kHead;
  const char* vpre8 = (const char*)p.cv + (size_t)b * p.c_vSeq + (size_t)kvh * p.c_vHead;
  const char* kslf8 = (const char*)p.sk + (size_t)(t + p.s_seq0) * p.s_kSeq + (size_t)kvh * p.s_kHead;
  const char* vslf8 = (const char*)p.sv + (size_t)(t + p.s_seq0) * p.s_vSeq + (size_t)kvh * p.s_vHead;

  // lane-constant parts of the DMA addresses
  int krow[KL], kchunk[KL], vrow[VL], vchunk[VL];
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    krow[i] = (wid * KL + i) * RPI + lane / CK;
    kchunk[i] = (lane % CK) ^ kswz<HD>(krow[i]);
  }
#pragma unroll
  for (int i = 0; i < VL; ++i) {
    vrow[i] = (wid * VL + i) * 8 + (lane >> 3);
    vchunk[i] = (lane & 7) ^ ((vrow[i] >> 1) & 7);
  }
  auto issue = [&](int tile, int slot) {
    if (F8) {
      // fp8 chunks land unswizzled: K chunk q = (key row q / CK8, 16 hd elements q % CK8), then
      // V^T chunk q = (hd row q / 4, 16 keys q % 4)
      char* base8 = ring8 + slot * STAGE8;
      const bool pre = tile < TP;
      const int k0 = pre ? tile * AKT : (tile - TP) * AKT;
      const int klen = pre ? p.n_cache : p.n_self;
      const char* kb = pre ? kpre8 : kslf8;
      const int64_t kpos = pre ? p.c_kPos : p.s_kPos;
      const char* vb = pre ? vpre8 : vslf8;
      const int64_t vr = pre ? p.c_vRow : p.s_vRow;
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const int q = (wid * KL + i) * 64 + lane;
        const int key = min(k0 + q / CK8, klen - 1);  // rows past the segment load a valid row (masked)
        __builtin_amdgcn_global_load_lds((const void*)(kb + (size_t)key * kpos + (q % CK8) * 16),
                                         LDS_PTR(base8 + (wid * KL + i) * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int q = (wid * VL + i) * 64 + lane;
        __builtin_amdgcn_global_load_lds((const void*)(vb + (size_t)(q >> 2) * vr + k0 + (q & 3) * 16),
                                         LDS_PTR(base8 + AKT * HD + (wid * VL + i) * 1024), 16, 0, 0);
      }
      return;
    }
    bf16_t* base = smem + slot * STAGE;
    const bool pre = tile < TP;
    const int k0 = pre ? tile * AKT : (tile - TP) * AKT;  // first key of the tile in its segment
    const int klen = pre ? p.n_cache : p.n_self;
    const bf16_t* kb = pre ? kpre : kslf;
    const int64_t kpos = pre ? p.c_kPos : p.s_kPos;
    const bf16_t* vb = pre ? vpre : vslf;
    const int64_t vr = pre ? p.c_vRow : p.s_vRow;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int key = min(k0 + krow[i], klen - 1);  // rows past the segment load a valid row (masked)
      __builtin_amdgcn_global_load_lds((const void*)(kb + (size_t)key * kpos + kchunk[i] * 8),
                                       LDS_PTR(base + (wid * KL + i) * 512), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VL; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(vb + (size_t)vrow[i] * vr + k0 + vchunk[i] * 8),
                                       LDS_PTR(base + KST + (wid * VL + i) * 512), 16, 0, 0);
  };

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

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (tb + s < te) issue(tb + s, s);

  for (int tile = tb; tile < te; ++tile) {
    const int it = tile - tb;
    if (tile + NS - 1 <= te)
      wait_vmcnt_le<(NS - 2) * LPW>();
    else
      wait_vmcnt_le<0>();
    // every wave's loads of this stage have landed, and every wave is done with the slot refilled below
    // (and, with fp8, with the working tile)
    lds_barrier();
    if (tile + NS - 1 < te) issue(tile + NS - 1, (it + NS - 1) % NS);
    const bf16_t* sK = F8 ? work : smem + (it % NS) * STAGE;
    const bf16_t* sV = sK + KST;
    if (F8) {  // convert the landed fp8 stage into the swizzled bf16 working tile
      const char* s8 = ring8 + (it % NS) * STAGE8;
      bf16_t* wK = work;
      bf16_t* wV = work + KST;
      for (int q = tid; q < AKT * CK8; q += NW * 64) {
        const uint4 in = *(const uint4*)(s8 + q * 16);
        uint4 lo, hi;
        fp8x16_to_bf16(in, lo, hi);
        const int r = q / CK8, c = 2 * (q % CK8);
        *(uint4*)&wK[r * HD + ((c ^ kswz<HD>(r)) << 3)] = lo;
        *(uint4*)&wK[r * HD + (((c + 1) ^ kswz<HD>(r)) << 3)] = hi;
      }
      for (int q = tid; q < HD * 4; q += NW * 64) {
        const uint4 in = *(const uint4*)(s8 + AKT * HD + q * 16);
        uint4 lo, hi;
        fp8x16_to_bf16(in, lo, hi);
        const int e = q >> 2, c = 2 * (q & 3), sw = (e >> 1) & 7;
        *(uint4*)&wV[e * AKT + ((c ^ sw) << 3)] = lo;
        *(uint4*)&wV[e * AKT + (((c + 1) ^ sw) << 3)] = hi;
      }
      lds_barrier_lds_only();
    }
    const bool pre = tile < TP;
    const int k0 = pre ? tile * AKT : (tile - TP) * AKT;
    const int klen = pre ? p.n_cache : p.n_self;

    // S^T = K Q^T : 4 key subtiles x NQ query subtiles, hd chunk by hd chunk.  Each chunk's K
    // fragments are read one chunk ahead of its MFMAs, into the other register set, and retired by
    // an explicit LDS-counter wait (the compiler's own waits treat the direct-to-LDS loads as
    // unordered with these reads and would also wait for the reads just issued).
    // (subtile j of this wave is S subtile kh * KS + j of the tile)
    floatx4 s[KS][NQ];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) s[ks][nq] = (floatx4){0.f, 0.f, 0.f, 0.f};
    auto read_k = [&](int c, bf16x8_t (&f)[KS]) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r = s_key(kh * KS + ks, col);
        f[ks] = *(const bf16x8_t*)&sK[r * HD + (((c * 4 + quad) ^ kswz<HD>(r)) << 3)];
      }
    };
    bf16x8_t kf[2][KS];
    read_k(0, kf[0]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 1 < NC) read_k(c + 1, kf[(c + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq)
          s[ks][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c & 1][ks], qf[nq][c], s[ks][nq], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V^T fragments are read while the softmax runs
    constexpr int HG = NH >= 2 ? 2 : 1;  // hd row blocks per V^T read group
    auto read_v = [&](int g, bf16x8_t (&f)[HG][C2]) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const int r = (g * HG + hh) * 16 + col;
        const int sw = (r >> 1) & 7;
#pragma unroll
        for (int c2 = 0; c2 < C2; ++c2)
          f[hh][c2] = *(const bf16x8_t*)&sV[r * AKT + ((((kh * C2 + c2) * 4 + quad) ^ sw) << 3)];
      }
    };
    bf16x8_t vf[2][HG][C2];
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    read_v(0, vf[0]);
    __builtin_amdgcn_sched_barrier(0);

    // Online softmax per query column in base-2 units: scores times scale * log2(e), so each
    // probability is one hardware exp2.  Masking runs only on tiles that need it (the segment's
    // last tile, or own keys under a causal mask); rows past the block (qok false) need none:
    // their query is zero, and their column is never written.
    const bool full = k0 + AKT <= klen && !(p.causal && !pre);
    bf16x8_t pb[C2][NQ];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      // raw scores; masked ones become -inf (exp2 of -inf is 0)
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[ks][nq][v]);
      } else {
        const int lim = (p.causal && !pre) ? qpos[nq] + p.causal_off : klen;  // last visible own key
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int kk = k0 + s_key(kh * KS + ks, quad * 4 + v);  // key within its segment
            const bool ok = (kk < klen) & (kk <= lim);
            const float sc = ok ? s[ks][nq][v] : -INFINITY;
            s[ks][nq][v] = sc;
            mx = fmaxf(mx, sc);
          }
      }
      mx *= scale2;  // the scale is positive: the max of the scaled scores
      // Raise the column's running max only when some lane saw a larger score: the test is a
      // wave vote, and the cross-lane max (two crossbar shuffles) runs only then -- after the
      // first tiles most tiles skip it.  lrun holds this lane's partial sum (its 16 keys of each
      // tile) against the column's common max; the quads' sums are added once at the end.
      if (__any(mx > mrun[nq])) {
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(mrun[nq], mx);
        const float corr = __builtin_amdgcn_exp2f(mrun[nq] - mnew);  // 0 while mrun is -inf
        lrun[nq] *= corr;
#pragma unroll
        for (int h = 0; h < NH; ++h) o[h][nq] *= corr;
        mrun[nq] = mnew;
      }
      const float mref = mrun[nq] == -INFINITY ? 0.f : mrun[nq];  // masked scores give exp2(-inf) = 0
      float sum = 0.f;
      float pv[KS][4];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[ks][nq][v], scale2, -mref));
          pv[ks][v] = e;
          sum += e;
        }
      lrun[nq] += sum;
#pragma unroll
      for (int c2 = 0; c2 < C2; ++c2) {
        uint4 w;
        w.x = pack_bf16x2(pv[2 * c2][0], pv[2 * c2][1]);
        w.y = pack_bf16x2(pv[2 * c2][2], pv[2 * c2][3]);
        w.z = pack_bf16x2(pv[2 * c2 + 1][0], pv[2 * c2 + 1][1]);
        w.w = pack_bf16x2(pv[2 * c2 + 1][2], pv[2 * c2 + 1][3]);
        pb[c2][nq] = *(bf16x8_t*)&w;
      }
    }

    // O^T += V^T P^T ; lane's 8 k-slots are keys 32c2 + 8quad + {0..7}: one 16-byte chunk.  V^T
    // fragments are read one group of hd row blocks ahead of their MFMAs.
#pragma unroll
    for (int g = 0; g < NH / HG; ++g) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
      if (g + 1 < NH / HG) read_v(g + 1, vf[(g + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh)
#pragma unroll
        for (int c2 = 0; c2 < C2; ++c2)
#pragma unroll
          for (int nq = 0; nq < NQ; ++nq)
            o[g * HG + hh][nq] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[g & 1][hh][c2], pb[c2][nq], o[g * HG + hh][nq], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the column's sum over its four quads of lanes
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    lrun[nq] += __shfl_xor(lrun[nq], 16, 64);
    lrun[nq] += __shfl_xor(lrun[nq], 32, 64);
  }
  if constexpr (KH == 2) {
    // Combine the two key halves of each query sub-block: wave kh = 1 leaves its (max, sum, O)
    // in LDS, wave kh = 0 rescales both to the common max and adds.  The ring is free once every
    // wave has passed the barrier (no loads are in flight after the last tile).
    constexpr int PER = NH * NQ * 4 + 2 * NQ;  // floats per lane
    float* xch = (float*)smem + (size_t)wq * PER * 64 + lane;
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int v = 0; v < 4; ++v) xch[((nq * NH + h) * 4 + v) * 64] = o[h][nq][v];
        xch[(NH * NQ * 4 + 2 * nq) * 64] = mrun[nq];
        xch[(NH * NQ * 4 + 2 * nq + 1) * 64] = lrun[nq];
      }
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      const float m1 = xch[(NH * NQ * 4 + 2 * nq) * 64], l1 = xch[(NH * NQ * 4 + 2 * nq + 1) * 64];
      const float M = fmaxf(mrun[nq], m1);
      const float f0 = mrun[nq] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[nq] - M);
      const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
      lrun[nq] = f0 * lrun[nq] + f1 * l1;
      mrun[nq] = M;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[h][nq][v] = f0 * o[h][nq][v] + f1 * xch[((nq * NH + h) * 4 + v) * 64];
    }
  }
  // write: lane holds query column col of subtile nq, hd rows h*16 + 4*quad + v
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    if (!qok[nq]) continue;
    const int rho = qb * QB + wq * QW + nq * 16 + col;
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
        part[HD] = mrun[nq] * 0.69314718055994531f;  // base-2 running max back in natural units
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
  // up to MS splits: every partial is loaded before any is combined (one memory round trip)
  constexpr int MS = 8, NU = (HD + 63) / 64;
  float ms_[MS], ls_[MS], vs_[MS][NU];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    if (s < n_splits) {
      const float* ps = part + s * (HD + 2);
      ms_[s] = ps[HD];
      ls_[s] = ps[HD + 1];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int e = lane + 64 * u;
        vs_[s][u] = e < HD ? ps[e] : 0.f;
      }
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s)
    if (s < n_splits) M = fmaxf(M, ms_[s]);
  for (int s = MS; s < n_splits; ++s) M = fmaxf(M, part[s * (HD + 2) + HD]);
  float L = 0.f, acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = 0.f;
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    if (s < n_splits) {
      const float f = ms_[s] == -INFINITY ? 0.f : __expf(ms_[s] - M);
      L += f * ls_[s];
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[u] += f * vs_[s][u];
    }
  }
  for (int s = MS; s < n_splits; ++s) {  // splits past MS, straight from memory
    const float* ps = part + s * (HD + 2);
    const float f = ps[HD] == -INFINITY ? 0.f : __expf(ps[HD] - M);
    L += f * ps[HD + 1];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
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

template <int HD, int QW, int NW, bool F8, int KH = 1>
static void run_attn(const AttnParams& p, int n_pairs, int n_qblocks, int n_splits, int tps, int ns, hipStream_t st) {
  const int total = n_pairs * n_qblocks * n_splits;
  const int grid = ((total + 7) / 8) * 8;
  if (ns == 2)
    k_attn_mfma<HD, QW, 2, NW, F8, KH><<<grid, NW * 64, 0, st>>>(p, n_pairs, n_qblocks, n_splits, tps);
  else if (ns == 4)
    k_attn_mfma<HD, QW, 4, NW, F8, KH><<<grid, NW * 64, 0, st>>>(p, n_pairs, n_qblocks, n_splits, tps);
  else
    k_attn_mfma<HD, QW, 3, NW, F8, KH><<<grid, NW * 64, 0, st>>>(p, n_pairs, n_qblocks, n_splits, tps);
  if (n_splits > 1) {
    const int rows_q = (p.Hq / p.Hkv) * p.rows_per_seq;
    const int waves = n_pairs * rows_q;
    k_attn_merge<HD><<<(waves + 3) / 4, 256, 0, st>>>(p, n_pairs, n_splits);
  }
}

bool attn_mfma_supported(int hd) { return hd == 32 || hd == 64 || hd == 128; }

// p.n_rows / rows_per_seq = sequence slots; p.part must hold n_pairs * rows_q * max_splits * (hd + 2)
// floats when max_splits > 1.  Key rows must be 16-byte aligned and V^T rows (c_vRow, s_vRow
// elements) multiples of 64 elements; n_cache >= 1 or n_self >= 1.
void launch_attn_mfma(const AttnParams& p, int max_splits, hipStream_t st, int force_splits, int force_qw,
                      int force_ns, int force_nw, int force_kh) {
  if (p.n_rows <= 0) return;
  const int n_seq = p.n_rows / p.rows_per_seq;
  const int n_pairs = n_seq * p.Hkv;
  const int rows_q = (p.Hq / p.Hkv) * p.rows_per_seq;
  // Measured.  8B shape (128 query rows per pair, 17 key tiles): one eight-wave block of 16-row
  // waves per pair, a two-stage ring and about one block per compute unit through key splits
  // beat four-wave blocks, wider waves and deeper rings.  Long prefixes (>= 64 key tiles,
  // >= 256 query rows per pair): one eight-wave block per pair covering all its query rows (32
  // per wave; 16 with fp8 K/V), so each key tile is streamed once per pair, and no key split
  // when the pairs alone fill the chip (8192-key prefix: 113 -> 83 ms of attention per step).
  const int n_tiles = (p.n_cache + AKT - 1) / AKT + (p.n_self + AKT - 1) / AKT;
  const bool long_kv = p.hd >= (p.kv8 ? 128 : 64) && rows_q >= 256 && n_tiles >= 64;
  // >= 128 query rows per pair: eight 16-row waves share each K/V stream (8B step: 2.12 -> 1.94 ms)
  const bool wide_q = p.hd >= (p.kv8 ? 128 : 64) && rows_q >= 128;
  // Key halves (four waves over 32 query rows, every key tile of the pair in one block, no key
  // split or merge launch once the blocks fill the chip) on request only: at the 8B step they
  // measured 1.77 ms of attention per step against 1.52 ms for the eight-wave blocks with key
  // splits -- with one wave per SIMD the score products' accumulation chains stay exposed.
  const bool kh2 = force_kh == 2 && !p.kv8 && (p.hd == 128 || p.hd == 64);
  const int QW = kh2 ? 16 : (force_qw == 16 || force_qw == 32) ? force_qw : (long_kv && !p.kv8 ? 32 : 16);
  const int NW = kh2 ? 4
                     : ((force_nw == 8 || (force_nw == 0 && (long_kv || wide_q))) && p.hd >= (p.kv8 ? 128 : 64)) ? 8
                                                                                                                   : 4;
  const int QB = (kh2 ? NW / 2 : NW) * QW;
  const int n_qblocks = (rows_q + QB - 1) / QB;
  int splits = 1;
  if (!p.causal && p.part) {
    // long: enough splits for about one block per compute unit; else about two blocks per
    // compute unit and at least two splits, at least 2 key tiles per split; key halves: no
    // split once the blocks cover three quarters of the compute units
    const int blocks = n_pairs * n_qblocks;
    const int want = kh2 ? (blocks >= 192 ? 1 : (256 + blocks - 1) / blocks)
                   : long_kv ? max(1, (256 + blocks - 1) / blocks)
                             : (NW == 8 ? max(2, (256 + blocks - 1) / blocks) : max(2, (512 + blocks - 1) / blocks));
    splits = min(min(want, max(1, n_tiles / 2)), max_splits);
    if (force_splits > 0) splits = min(force_splits, max_splits);
    if (splits < 1) splits = 1;
  }
  const int tps = (n_tiles + splits - 1) / splits;
  splits = (n_tiles + tps - 1) / tps;
  if (splits < 1) splits = 1;
  const int ns = (force_ns >= 2 && force_ns <= 4) ? force_ns : (kh2 ? 4 : 2);
  if (kh2) {
    if (p.hd == 128) run_attn<128, 16, 4, false, 2>(p, n_pairs, n_qblocks, splits, tps, ns, st);
    else run_attn<64, 16, 4, false, 2>(p, n_pairs, n_qblocks, splits, tps, ns, st);
    return;
  }
#define GO(H, Q, W) run_attn<H, Q, W, false>(p, n_pairs, n_qblocks, splits, tps, ns, st)
#define GO8(H, Q, W) run_attn<H, Q, W, true>(p, n_pairs, n_qblocks, splits, tps, ns, st)
  if (p.kv8) {  // fp8 keys and values (head sizes 64 and 128)
    if (p.hd == 128) {
      if (NW == 8) {
        if (QW == 16) GO8(128, 16, 8); else GO8(128, 32, 8);
      } else {
        if (QW == 16) GO8(128, 16, 4); else GO8(128, 32, 4);
      }
    } else {
      if (QW == 16) GO8(64, 16, 4); else GO8(64, 32, 4);
    }
    return;
  }
  if (p.hd == 128) {
    if (NW == 8) {
      if (QW == 16) GO(128, 16, 8); else GO(128, 32, 8);
    } else {
      if (QW == 16) GO(128, 16, 4); else GO(128, 32, 4);
    }
  } else if (p.hd == 64) {
    if (NW == 8) {
      if (QW == 16) GO(64, 16, 8); else GO(64, 32, 8);
    } else {
      if (QW == 16) GO(64, 16, 4); else GO(64, 32, 4);
    }
  } else {
    if (QW == 16) GO(32, 16, 4); else GO(32, 32, 4);
  }
#undef GO
#undef GO8
}

}  // namespace alodlm
