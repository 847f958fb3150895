/* Seeded synthetic inputs: one counter-based generator, defined here.
 *
 * Test and benchmark infrastructure only. It holds none of the decode step's
 * arithmetic: it draws numbers and writes them into documented storage
 * formats. Both the oracle (host, fx_host.c) and the GPU inputs (device,
 * fx_gpu.hip) are filled from these definitions, and each implementation
 * reproduces them bit for bit (integer operations, one IEEE fp32 multiply).
 *
 * Definitions
 *   GAMMA            = 0x9E3779B97F4A7C15 (SplitMix64 increment)
 *   mix64(z)         = SplitMix64 output finaliser (Steele, Lea, Flood 2014;
 *                      constants of Stafford's "Mix13"):
 *                      z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                      z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
 *   stream(key, n)   = mix64(key + (n + 1) * GAMMA), i.e. the n-th output
 *                      (0-based) of a SplitMix64 generator seeded with key
 *   key(seed, tag)   = mix64(stream(seed, 0) ^ tag)
 *   tag(kind, l, a, b) = kind << 56 | l << 40 | a << 20 | b
 *   normal(key, i, sigma): the twelve 16-bit fields of stream(key, 3i),
 *                      stream(key, 3i+1), stream(key, 3i+2) are summed to s;
 *                      z = float(2 s - 786420); value = z * (sigma * 2^-17)
 *                      in fp32. This is the Irwin-Hall(12) approximation of
 *                      a normal variate: mean 0, variance sigma^2 (1 - 2^-32),
 *                      support +-6 sigma.
 *   bf16(value)      = round-to-nearest-even of the fp32 bit pattern to its
 *                      upper 16 bits.
 *   uniform(key, i, lo, hi) = lo + ((stream(key, i) >> 32) * (hi - lo + 1) >> 32)
 *   permutation(n, key): a = [0, n); for i = n-1 .. 1:
 *                      j = uniform(key, n-1-i, 0, i); swap(a[i], a[j])
 */
#ifndef FX_H
#define FX_H
#include <stdint.h>
#include <stddef.h>

#define FX_GAMMA 0x9E3779B97F4A7C15ull

enum fx_kind {
  FX_EMBED = 1, FX_ATTN_NORM = 2, FX_WQKV = 3, FX_WO = 4, FX_FFN_NORM = 5,
  FX_ROUTER = 6, FX_GATE = 7, FX_UP = 8, FX_DOWN = 9, FX_FINAL_NORM = 10,
  FX_LM_HEAD = 11, FX_KCACHE = 12, FX_VCACHE = 13, FX_TOKEN = 14, FX_CTX = 15,
  FX_PERM = 16
};

#ifdef __cplusplus
extern "C" {
#endif
uint64_t fx_mix64(uint64_t z);
uint64_t fx_stream(uint64_t key, uint64_t n);
uint64_t fx_tag(uint64_t kind, uint64_t layer, uint64_t a, uint64_t b);
uint64_t fx_key(uint64_t seed, uint64_t tag);
float    fx_normal_f32(uint64_t key, uint64_t i, float sigma);
uint16_t fx_bf16_rne(float v);
uint32_t fx_uniform(uint64_t key, uint64_t i, uint32_t lo, uint32_t hi);
/* dst[j] = bf16(normal(key, i0 + j, sigma)), j < n. OpenMP over j. */
void fx_fill_normal_bf16(uint16_t* dst, uint64_t key, uint64_t i0, uint64_t n, float sigma);
void fx_fill_const_bf16(uint16_t* dst, uint64_t n, uint16_t bits);
void fx_permutation(int32_t* out, int32_t n, uint64_t key);
void fx_uniform_fill(uint32_t* out, uint64_t key, uint64_t i0, uint64_t n, uint32_t lo, uint32_t hi);
int  fx_threads(void);
#ifdef __cplusplus
}
#endif
#endif
