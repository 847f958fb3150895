// Device implementation of the generator defined in fx.h, used to fill
// GPU-resident synthetic inputs in place (weights of tens of GB, paged KV).
// Test and benchmark infrastructure only; bit-identical to fx_host.c by
// construction (integer arithmetic and one IEEE fp32 multiply) and checked
// against it on sampled indices by the GPU tests.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "fx.h"

namespace {

__device__ __forceinline__ uint64_t d_mix64(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27; z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t d_stream(uint64_t key, uint64_t n) {
  return d_mix64(key + (n + 1) * FX_GAMMA);
}
__device__ __forceinline__ uint64_t d_key(uint64_t seed, uint64_t tag) {
  return d_mix64(d_stream(seed, 0) ^ tag);
}
__device__ __forceinline__ uint32_t d_sum16(uint64_t w) {
  return (uint32_t)(w & 0xFFFF) + (uint32_t)((w >> 16) & 0xFFFF) +
         (uint32_t)((w >> 32) & 0xFFFF) + (uint32_t)(w >> 48);
}
__device__ __forceinline__ uint16_t d_normal_bf16(uint64_t key, uint64_t i, float c) {
  uint32_t s = d_sum16(d_stream(key, 3 * i)) + d_sum16(d_stream(key, 3 * i + 1)) +
               d_sum16(d_stream(key, 3 * i + 2));
  float z = (float)((int32_t)(2 * s) - 786420);
  float v = __fmul_rn(z, c);
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void k_fill_normal(uint16_t* dst, uint64_t key, uint64_t i0, uint64_t n, float c) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    dst[j] = d_normal_bf16(key, i0 + j, c);
}

// dst is [n_layers][n_sub][per]; matrix (l, e) uses key(seed, tag(kind, l0 + l, e, 0)).
__global__ void k_fill_stack(uint16_t* dst, uint64_t seed, uint64_t kind, uint32_t l0,
                             uint32_t n_sub, uint64_t per, uint64_t total, float c) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < total; j += stride) {
    uint64_t m = j / per, i = j - m * per;
    uint64_t l = m / n_sub, e = m - l * n_sub;
    uint64_t tag = (kind << 56) | ((l0 + l) << 40) | (e << 20);
    dst[j] = d_normal_bf16(d_key(seed, tag), i, c);
  }
}

__global__ void k_fill_const(uint16_t* dst, uint64_t n, uint16_t bits) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    dst[j] = bits;
}

// Paged KV of one sequence b in the documented pool format: for page p,
// layer l, kv head g the block of 2*PT*d bf16 at
// p*page_stride + l*layer_stride + g*2*PT*d holds K as [slot][dim] followed
// by V as [dim][slot]. Token t sits in page page_table[t / PT], slot t % PT.
// Element (t, i) of K (V) of (l, g) is normal(key(seed, tag(KCACHE (VCACHE),
// l, b, g)), t*d + i, 1). Slots at t < t0 or t >= ctx are left untouched.
__global__ void k_fill_kv(uint16_t* pool, const int32_t* page_row, uint64_t seed, uint32_t b,
                          uint32_t t0, uint32_t ctx, uint32_t n_pg, uint32_t L, uint32_t Hkv, uint32_t d,
                          uint32_t PT, uint64_t total, float c) {
  const uint64_t blk = 2ull * PT * d;
  const uint64_t layer_stride = (uint64_t)Hkv * blk;
  const uint64_t page_stride = (uint64_t)L * layer_stride;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < total; j += stride) {
    uint64_t e = j % blk; uint64_t r = j / blk;
    uint32_t g = (uint32_t)(r % Hkv); r /= Hkv;
    uint32_t l = (uint32_t)(r % L); r /= L;
    uint32_t pg = (uint32_t)r;  // logical page index within the sequence
    // block layout (the library's KV pool format, operand order): K element
    // ((dim/32*4 + dim%32/8)*16 + s)*8 + dim%8, then V element
    // ((dim/32*4 + s/4)*16 + dim%16)*8 + (dim%32/16)*4 + s%4
    uint32_t kv, s, i;
    if (e < (uint64_t)PT * d) {
      kv = 0;
      const uint32_t c = (uint32_t)(e / 8), e8 = (uint32_t)(e % 8), q = c / 16;
      s = c % 16;
      i = (q / 4) * 32 + (q % 4) * 8 + e8;
    } else {
      kv = 1;
      const uint64_t e2 = e - (uint64_t)PT * d;
      const uint32_t c = (uint32_t)(e2 / 8), e8 = (uint32_t)(e2 % 8), q = c / 16, r = c % 16;
      s = (q % 4) * 4 + (e8 % 4);
      i = (q / 4) * 32 + (e8 / 4) * 16 + r;
    }
    uint32_t t = pg * PT + s;
    if (t < t0 || t >= ctx || pg >= n_pg) continue;
    uint64_t kind = kv ? (uint64_t)FX_VCACHE : (uint64_t)FX_KCACHE;
    uint64_t tag = (kind << 56) | ((uint64_t)l << 40) | ((uint64_t)b << 20) | g;
    uint64_t phys = (uint64_t)page_row[pg];
    pool[phys * page_stride + (uint64_t)l * layer_stride + (uint64_t)g * blk + e] =
        d_normal_bf16(d_key(seed, tag), (uint64_t)t * d + i, c);
  }
}

inline unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  return (unsigned)(g > 65536 ? 65536 : (g == 0 ? 1 : g));
}

}  // namespace

extern "C" {

int fx_gpu_fill_normal_bf16(void* dst, uint64_t key, uint64_t i0, uint64_t n, float sigma,
                            void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_normal, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)dst, key, i0, n, sigma * 7.62939453125e-06f);
  return (int)hipGetLastError();
}

int fx_gpu_fill_stack_bf16(void* dst, uint64_t seed, uint32_t kind, uint32_t l0,
                           uint32_t n_layers, uint32_t n_sub, uint64_t per, float sigma,
                           void* stream) {
  uint64_t total = (uint64_t)n_layers * n_sub * per;
  if (total == 0) return 0;
  hipLaunchKernelGGL(k_fill_stack, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)dst, seed, (uint64_t)kind, l0, n_sub, per, total,
                     sigma * 7.62939453125e-06f);
  return (int)hipGetLastError();
}

int fx_gpu_fill_const_bf16(void* dst, uint64_t n, uint16_t bits, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_fill_const, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)dst, n, bits);
  return (int)hipGetLastError();
}

// page_row: device pointer to this sequence's row of the page table (n_pg entries).
int fx_gpu_fill_kv(void* pool, const int32_t* page_row, uint64_t seed, uint32_t b,
                   uint32_t t0, uint32_t ctx, uint32_t n_pg, uint32_t L, uint32_t Hkv, uint32_t d,
                   uint32_t PT, void* stream) {
  uint64_t need = ((uint64_t)ctx + PT - 1) / PT;
  if (need > n_pg) return -1;
  uint64_t total = need * L * Hkv * 2ull * PT * d;
  if (total == 0) return 0;
  hipLaunchKernelGGL(k_fill_kv, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)pool, page_row, seed, b, t0, ctx, (uint32_t)need, L, Hkv, d, PT,
                     total, 1.0f * 7.62939453125e-06f);
  return (int)hipGetLastError();
}

}  // extern "C"
