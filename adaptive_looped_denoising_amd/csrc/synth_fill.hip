// Device fill of seeded synthetic tensors (workload generation; not part of the method).
// Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw (SC'11), mapped to the
// Irwin-Hall(4) value times a scale in one fp32 multiply; see include/alodlm_synth.h.
#include "../../include/alodlm_synth.h"
#include "common.h"
#include "launch.h"

namespace alodlm {

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ __forceinline__ float ih4_value(uint64_t i, uint32_t seed, uint32_t tensor, float scale) {
  const uint64_t n = i >> 1;
  uint32_t c[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
  philox4x32_10(c, seed, tensor);
  const uint32_t a = (i & 1) ? c[2] : c[0];
  const uint32_t b = (i & 1) ? c[3] : c[1];
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
__global__ __launch_bounds__(256) void k_fill_kv_synth(T* __restrict__ base, int B, int Hkv, int P, int P_max,
                                                       int hd, uint32_t seed, uint32_t tensor, float scale) {
  const uint64_t n = (uint64_t)B * Hkv * P * hd;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t k = (uint64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += stride) {
    const uint64_t e = k % hd;
    const uint64_t j = (k / hd) % P;
    const uint64_t bh = k / ((uint64_t)hd * P);
    base[(bh * P_max + j) * hd + e] = from_f<T>(ih4_value(k, seed, tensor, scale));
  }
}

void launch_fill_kv_synth(int dtype, void* slot_base, int B, int Hkv, int P, int P_max, int hd, uint32_t seed,
                          uint32_t tensor, float scale, hipStream_t st) {
  const uint64_t n = (uint64_t)B * Hkv * P * hd;
  if (!n) return;
  const unsigned grid = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (dtype == DT_BF16)
    k_fill_kv_synth<bf16_t><<<grid, 256, 0, st>>>((bf16_t*)slot_base, B, Hkv, P, P_max, hd, seed, tensor, scale);
  else
    k_fill_kv_synth<float><<<grid, 256, 0, st>>>((float*)slot_base, B, Hkv, P, P_max, hd, seed, tensor, scale);
}

__global__ void k_fill_u8(uint8_t* dst, size_t n, uint8_t v) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = v;
}
__global__ void k_copy_u8(uint8_t* dst, const uint8_t* src, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}
void launch_fill_u8(uint8_t* dst, size_t n, uint8_t v, hipStream_t st) {
  if (n) k_fill_u8<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(dst, n, v);
}
void launch_copy_avail(uint8_t* dst, const uint8_t* src, size_t n, hipStream_t st) {
  if (n) k_copy_u8<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(dst, src, n);
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
