/*
 * Host half of the seeded input generator (no arithmetic of the method).
 *
 * Every synthetic tensor is a pure function of (seed, tensor id, element
 * index), drawn from the counter-based generator Philox4x32-10 as published
 * by Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3" (SC'11): a 128-bit counter and a 64-bit key go through ten
 * rounds of two 32x32->64 multiplies, with the key bumped by the Weyl
 * constants between rounds.  The GPU library carries its own implementation
 * of the same published definition for tensors too large to upload; the
 * two are compared element for element in the tests.
 *
 * Value maps (all exact integer or single-rounding fp32 arithmetic so that
 * any correct implementation reproduces them bit for bit):
 *   ih4    : z = sum of four 16-bit uniforms - 131070 (Irwin-Hall of order 4,
 *            std 2^16/sqrt(3) = 37837.2), value = fp32(z) * fp32(scale),
 *            optionally rounded to bfloat16 (round to nearest even).
 *            Element i uses Philox block i/2: words (x0,x1) if i is even,
 *            (x2,x3) if odd.
 *   u32    : raw 32-bit words, element i = word i%4 of block i/4.
 * Counter of block n = (n mod 2^32, n div 2^32, 0, 0); key = (seed, tensor).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void alodlm_synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                                uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void block(uint64_t n, uint32_t seed, uint32_t tensor, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
  uint32_t key[2] = {seed, tensor};
  alodlm_synth_philox4x32_10(ctr, key, out);
}

static inline int32_t ih4(uint32_t a, uint32_t b) {
  return (int32_t)((a & 0xFFFFu) + (a >> 16) + (b & 0xFFFFu) + (b >> 16)) - 131070;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* fp32 output: out[k] = value of element start+k. */
void alodlm_synth_ih4_f32(float* out, uint64_t start, uint64_t n, uint32_t seed,
                          uint32_t tensor, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k) {
    uint64_t i = start + (uint64_t)k;
    uint32_t x[4];
    block(i >> 1, seed, tensor, x);
    int32_t z = (i & 1) ? ih4(x[2], x[3]) : ih4(x[0], x[1]);
    out[k] = (float)z * scale;
  }
}

/* bfloat16 output (bit pattern), RNE from the fp32 value above. */
void alodlm_synth_ih4_bf16(uint16_t* out, uint64_t start, uint64_t n, uint32_t seed,
                           uint32_t tensor, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k) {
    uint64_t i = start + (uint64_t)k;
    uint32_t x[4];
    block(i >> 1, seed, tensor, x);
    int32_t z = (i & 1) ? ih4(x[2], x[3]) : ih4(x[0], x[1]);
    out[k] = f32_to_bf16_rne((float)z * scale);
  }
}

/* Raw words: out[k] = word (start+k)%4 of block (start+k)/4. */
void alodlm_synth_u32(uint32_t* out, uint64_t start, uint64_t n, uint32_t seed, uint32_t tensor) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < (int64_t)n; ++k) {
    uint64_t i = start + (uint64_t)k;
    uint32_t x[4];
    block(i >> 2, seed, tensor, x);
    out[k] = x[i & 3];
  }
}
