// Device-side helpers shared by the gfx950 kernels of the looped denoising step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace alodlm {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
// Round to nearest even (inputs are finite).
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// OCP FP8 E4M3 storage byte (sign, 4 exponent bits with bias 7, 3 fraction bits, largest finite
// 448).  Conversion from float: saturate to +-448, then the hardware's round to nearest even.
struct fp8_t {
  uint8_t b;
};
template <> __device__ __forceinline__ fp8_t from_f<fp8_t>(float v) {
  const float c = __builtin_amdgcn_fmed3f(v, 448.0f, -448.0f);
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false);
  fp8_t r;
  r.b = (uint8_t)(w & 0xFF);
  return r;
}
__device__ __forceinline__ float to_f(fp8_t v) { return __builtin_amdgcn_cvt_f32_fp8((int)v.b, 0); }

// LDS address operand of the direct global->LDS loads (each lane's bytes land at M0 + lane * size).
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt constraining only the vector-memory counter to <= N (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without the release/acquire fence of __syncthreads() (which would wait for
// every load in flight, including the prefetched pipeline stages).  Callers order their own
// memory operations with explicit waits; the empty asm keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier once this wave's LDS accesses have completed (a wait on the LDS counter only:
// vector-memory loads in flight, such as prefetched stages, stay in flight).  gfx9 s_waitcnt
// encoding: vmcnt and expcnt at their maxima, lgkmcnt = 0.
__device__ __forceinline__ void lds_barrier_lds_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum with a fixed reduction order (deterministic); red holds NT/64 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}

// Streaming softmax statistics of a set of logits z: m = max z, S = sum e^(z-m),
// T = sum (z-m) e^(z-m), idx = argmax (lowest index among equal maxima).
// Entropy = ln S - T/S, log-sum-exp = m + ln S.
struct SoftStat {
  float m, S, T;
  int idx;
};

__device__ __forceinline__ SoftStat softstat_empty() {
  SoftStat s;
  s.m = -INFINITY;
  s.S = 0.f;
  s.T = 0.f;
  s.idx = 0x7FFFFFFF;
  return s;
}

__device__ __forceinline__ SoftStat softstat_merge(const SoftStat& a, const SoftStat& b) {
  if (a.S == 0.f) return b;
  if (b.S == 0.f) return a;
  SoftStat r;
  r.m = fmaxf(a.m, b.m);
  const float da = a.m - r.m, db = b.m - r.m;
  const float ea = __expf(da), eb = __expf(db);
  r.S = a.S * ea + b.S * eb;
  r.T = (a.T + da * a.S) * ea + (b.T + db * b.S) * eb;
  r.idx = a.m > b.m ? a.idx : (b.m > a.m ? b.idx : min(a.idx, b.idx));
  return r;
}

// Gumbel-max draw of a set of logits: the largest z + g (g Gumbel noise) and its column,
// lowest column among equal values; an empty set has g = -inf and idx = INT_MAX.  The struct is
// the stored form; in registers the pair is kept as two scalars and merged with gstat_take
// (merging struct copies lets the compiler select between their addresses, i.e. put them in
// scratch memory).
struct GStat {
  float g;
  int idx;
};

// (g, idx) <- the better of (g, idx) and (og, oidx).
__device__ __forceinline__ void gstat_take(float& g, int& idx, float og, int oidx) {
  const bool tb = og > g || (og == g && oidx < idx);
  g = tb ? og : g;
  idx = tb ? oidx : idx;
}

// Merge of (g, idx) across the lanes of groups of 2 * o_max lanes (xor butterflies 1 .. o_max).
template <int O_MAX>
__device__ __forceinline__ void gstat_reduce_xor(float& g, int& idx) {
#pragma unroll
  for (int o = 1; o <= O_MAX; o <<= 1) {
    const float og = __shfl_xor(g, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    gstat_take(g, idx, og, oi);
  }
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC'11) on counter (c0, c1, c2, c3), in place,
// with key (k0, k1): ten rounds of two 32x32->64 multiplies by the Philox constants, the key
// bumped by the Weyl constants between rounds.  Scalar words (no array) so that callers can pick
// words with selects without the compiler placing them in scratch memory.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// Gumbel noise of one 32-bit draw x: u = (floor(x / 2^9) + 1/2) / 2^23 (exact in fp32, inside
// (0, 1)), g = -ln(-ln u).
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  const float u = ((float)(x >> 9) + 0.5f) * 1.1920928955078125e-07f;
  return -logf(-logf(u));
}


__device__ __forceinline__ SoftStat softstat_shfl_xor(const SoftStat& s, int o) {
  SoftStat r;
  r.m = __shfl_xor(s.m, o, 64);
  r.S = __shfl_xor(s.S, o, 64);
  r.T = __shfl_xor(s.T, o, 64);
  r.idx = __shfl_xor(s.idx, o, 64);
  return r;
}

}  // namespace alodlm
