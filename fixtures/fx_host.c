/* Host implementation of the generator defined in fx.h (the definition). */
#include "fx.h"
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

uint64_t fx_mix64(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27; z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
uint64_t fx_stream(uint64_t key, uint64_t n) { return fx_mix64(key + (n + 1) * FX_GAMMA); }
uint64_t fx_tag(uint64_t kind, uint64_t layer, uint64_t a, uint64_t b) {
  return (kind << 56) | (layer << 40) | (a << 20) | b;
}
uint64_t fx_key(uint64_t seed, uint64_t tag) { return fx_mix64(fx_stream(seed, 0) ^ tag); }

static inline uint32_t sum16(uint64_t w) {
  return (uint32_t)(w & 0xFFFF) + (uint32_t)((w >> 16) & 0xFFFF) +
         (uint32_t)((w >> 32) & 0xFFFF) + (uint32_t)(w >> 48);
}
float fx_normal_f32(uint64_t key, uint64_t i, float sigma) {
  uint32_t s = sum16(fx_stream(key, 3 * i)) + sum16(fx_stream(key, 3 * i + 1)) +
               sum16(fx_stream(key, 3 * i + 2));
  float z = (float)((int32_t)(2 * s) - 786420);
  float c = sigma * 7.62939453125e-06f; /* sigma * 2^-17, exact scaling */
  return z * c;
}
uint16_t fx_bf16_rne(float v) {
  uint32_t u; memcpy(&u, &v, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
uint32_t fx_uniform(uint64_t key, uint64_t i, uint32_t lo, uint32_t hi) {
  uint64_t u = fx_stream(key, i) >> 32;
  uint64_t span = (uint64_t)hi - (uint64_t)lo + 1;
  return lo + (uint32_t)((u * span) >> 32);
}
void fx_fill_normal_bf16(uint16_t* dst, uint64_t key, uint64_t i0, uint64_t n, float sigma) {
  long long nn = (long long)n;
#pragma omp parallel for schedule(static)
  for (long long j = 0; j < nn; ++j)
    dst[j] = fx_bf16_rne(fx_normal_f32(key, i0 + (uint64_t)j, sigma));
}
void fx_fill_const_bf16(uint16_t* dst, uint64_t n, uint16_t bits) {
  for (uint64_t j = 0; j < n; ++j) dst[j] = bits;
}
void fx_permutation(int32_t* out, int32_t n, uint64_t key) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i >= 1; --i) {
    uint32_t j = fx_uniform(key, (uint64_t)(n - 1 - i), 0, (uint32_t)i);
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}
void fx_uniform_fill(uint32_t* out, uint64_t key, uint64_t i0, uint64_t n, uint32_t lo, uint32_t hi) {
  for (uint64_t j = 0; j < n; ++j) out[j] = fx_uniform(key, i0 + j, lo, hi);
}
int fx_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
