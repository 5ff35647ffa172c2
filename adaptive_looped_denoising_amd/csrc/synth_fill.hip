// Device fill of seeded synthetic tensors (workload generation; not part of the method).
// Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw (SC'11), mapped to the
// Irwin-Hall(4) value times a scale in one fp32 multiply; see include/alodlm_synth.h.
#include "../../include/alodlm_synth.h"
#include "common.h"
#include "launch.h"

namespace alodlm {

__device__ __forceinline__ float ih4_value(uint64_t i, uint32_t seed, uint32_t tensor, float scale) {
  const uint64_t n = i >> 1;
  uint32_t c0 = (uint32_t)n, c1 = (uint32_t)(n >> 32), c2 = 0u, c3 = 0u;
  philox4x32_10(c0, c1, c2, c3, seed, tensor);
  const uint32_t a = (i & 1) ? c2 : c0;
  const uint32_t b = (i & 1) ? c3 : c1;
  const int32_t z = (int32_t)((a & 0xFFFFu) + (a >> 16) + (b & 0xFFFFu) + (b >> 16)) - 131070;
  return __fmul_rn((float)z, scale);
}

template <typename T>
__global__ __launch_bounds__(256) void k_synth_fill(T* __restrict__ dst, uint64_t start, uint64_t n, uint32_t seed,
                                                    uint32_t tensor, float scale, float offset) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t k = (uint64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += stride)
    dst[k] = from_f<T>(scale == 0.f ? offset : ih4_value(start + k, seed, tensor, scale));
}

// Cache slot [B][Hkv][P_max][hd]: element (b, h, j, e) = draw ((b*Hkv + h)*P + j)*hd + e.
template <typename T>
__global__ __launch_bounds__(256) void k_fill_kv_synth(T* __restrict__ base, int B, int Hkv, int P, int P_pitch,
                                                       int hd, uint32_t seed, uint32_t tensor, float scale,
                                                       int transposed) {
  const uint64_t n = (uint64_t)B * Hkv * P * hd;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t k = (uint64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += stride) {
    const uint64_t e = k % hd;
    const uint64_t j = (k / hd) % P;
    const uint64_t bh = k / ((uint64_t)hd * P);
    const uint64_t o = transposed ? (bh * hd + e) * P_pitch + j : (bh * P_pitch + j) * hd + e;
    base[o] = from_f<T>(ih4_value(k, seed, tensor, scale));
  }
}

void launch_fill_kv_synth(int dtype, void* slot_base, int B, int Hkv, int P, int P_pitch, int hd, uint32_t seed,
                          uint32_t tensor, float scale, bool transposed, hipStream_t st) {
  const uint64_t n = (uint64_t)B * Hkv * P * hd;
  if (!n) return;
  const unsigned grid = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (dtype == DT_FP8)  // the float32 draw rounded once to E4M3
    k_fill_kv_synth<fp8_t><<<grid, 256, 0, st>>>((fp8_t*)slot_base, B, Hkv, P, P_pitch, hd, seed, tensor, scale,
                                                 transposed ? 1 : 0);
  else if (dtype == DT_BF16)
    k_fill_kv_synth<bf16_t><<<grid, 256, 0, st>>>((bf16_t*)slot_base, B, Hkv, P, P_pitch, hd, seed, tensor, scale,
                                                  transposed ? 1 : 0);
  else
    k_fill_kv_synth<float><<<grid, 256, 0, st>>>((float*)slot_base, B, Hkv, P, P_pitch, hd, seed, tensor, scale,
                                                 transposed ? 1 : 0);
}

// One thread per (b, kvh, j, e): walks the planes of its element, copying the source plane's
// value into every plane above the position's available depth.
template <typename T>
__global__ __launch_bounds__(256) void k_materialize_depth(T* __restrict__ k0, T* __restrict__ v0,
                                                           int64_t plane_elems, int k_max, int B, int Hkv, int j0,
                                                           int n_pos, int P_pitch, int hd,
                                                           const uint8_t* __restrict__ avail, int av_pitch) {
  const uint64_t n = (uint64_t)B * Hkv * n_pos * hd;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t k = (uint64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += stride) {
    const uint64_t e = k % hd;
    const uint64_t j = j0 + (k / hd) % n_pos;
    const uint64_t bh = k / ((uint64_t)hd * n_pos);
    const int b = (int)(bh / Hkv);
    const int a = max(1, min(k_max, (int)avail[(size_t)b * av_pitch + j]));
    if (a >= k_max) continue;
    const uint64_t ok = (bh * P_pitch + j) * hd + e;      // K layout
    const uint64_t ov = (bh * hd + e) * P_pitch + j;      // transposed V layout
    const T kv = k0[(uint64_t)(a - 1) * plane_elems + ok];
    const T vv = v0[(uint64_t)(a - 1) * plane_elems + ov];
    for (int pl = a; pl < k_max; ++pl) {
      k0[(uint64_t)pl * plane_elems + ok] = kv;
      v0[(uint64_t)pl * plane_elems + ov] = vv;
    }
  }
}

void launch_materialize_depth(int dtype, void* k_plane0, void* v_plane0, int64_t plane_elems, int k_max, int B,
                              int Hkv, int j0, int n_pos, int P_pitch, int hd, const uint8_t* avail, int av_pitch,
                              hipStream_t st) {
  const uint64_t n = (uint64_t)B * Hkv * n_pos * hd;
  if (!n || k_max < 2) return;
  const unsigned grid = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (dtype == DT_FP8)
    k_materialize_depth<fp8_t><<<grid, 256, 0, st>>>((fp8_t*)k_plane0, (fp8_t*)v_plane0, plane_elems, k_max, B,
                                                     Hkv, j0, n_pos, P_pitch, hd, avail, av_pitch);
  else if (dtype == DT_BF16)
    k_materialize_depth<bf16_t><<<grid, 256, 0, st>>>((bf16_t*)k_plane0, (bf16_t*)v_plane0, plane_elems, k_max, B,
                                                      Hkv, j0, n_pos, P_pitch, hd, avail, av_pitch);
  else
    k_materialize_depth<float><<<grid, 256, 0, st>>>((float*)k_plane0, (float*)v_plane0, plane_elems, k_max, B, Hkv,
                                                     j0, n_pos, P_pitch, hd, avail, av_pitch);
}

template <typename T>
__global__ __launch_bounds__(256) void k_read_v_rows(const T* __restrict__ slot, int b, int Hkv, int P_pitch, int hd,
                                                     int j0, int n, T* __restrict__ dst) {
  const size_t total = (size_t)Hkv * n * hd;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int e = (int)(i % hd);
  const int jj = (int)((i / hd) % n);
  const int h = (int)(i / ((size_t)hd * n));
  dst[i] = slot[(((size_t)b * Hkv + h) * hd + e) * P_pitch + j0 + jj];
}

void launch_read_v_rows(int dtype, const void* slot_base, int b, int Hkv, int P_pitch, int hd, int j0, int n,
                        void* dst, hipStream_t st) {
  const size_t total = (size_t)Hkv * n * hd;
  if (!total) return;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (dtype == DT_FP8)
    k_read_v_rows<fp8_t><<<grid, 256, 0, st>>>((const fp8_t*)slot_base, b, Hkv, P_pitch, hd, j0, n, (fp8_t*)dst);
  else if (dtype == DT_BF16)
    k_read_v_rows<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)slot_base, b, Hkv, P_pitch, hd, j0, n, (bf16_t*)dst);
  else
    k_read_v_rows<float><<<grid, 256, 0, st>>>((const float*)slot_base, b, Hkv, P_pitch, hd, j0, n, (float*)dst);
}

__global__ void k_fill_u8(uint8_t* dst, size_t n, uint8_t v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = v;
}
// dst[b * pitch + j0 + j] = min(src ? src[b * n + j] : v, cap) for b < B, j < n
__global__ void k_set_avail(uint8_t* dst, int pitch, int j0, int B, int n, const uint8_t* src, uint8_t v,
                            uint8_t cap) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)B * n) return;
  const size_t b = i / n, j = i % n;
  const uint8_t a = src ? src[i] : v;
  dst[b * pitch + j0 + j] = a < cap ? a : cap;
}
void launch_set_avail(uint8_t* dst, int pitch, int j0, int B, int n, const uint8_t* src, uint8_t v, uint8_t cap,
                      hipStream_t st) {
  const size_t total = (size_t)B * n;
  if (total) k_set_avail<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(dst, pitch, j0, B, n, src, v, cap);
}

}  // namespace alodlm

extern "C" int alodlm_synth_fill(void* dst, int32_t dtype, uint64_t start, uint64_t n, uint32_t seed,
                                 uint32_t tensor, float scale, float offset, void* hip_stream) {
  using namespace alodlm;
  if (!dst || (dtype != DT_BF16 && dtype != DT_FP32)) return -1;
  if (!n) return 0;
  hipStream_t st = (hipStream_t)hip_stream;
  const unsigned grid = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (dtype == DT_BF16)
    k_synth_fill<bf16_t><<<grid, 256, 0, st>>>((bf16_t*)dst, start, n, seed, tensor, scale, offset);
  else
    k_synth_fill<float><<<grid, 256, 0, st>>>((float*)dst, start, n, seed, tensor, scale, offset);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
