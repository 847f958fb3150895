// Device helpers of the megakernel: bf16 unpacking, wave reductions, tagged
// (epoch-stamped) activation words and the bounded spin loops on them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.hpp"

namespace mk {
namespace dev {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));

constexpr float NEG_INF = -__builtin_inff();

// The thread index read through an opaque move. Values derived from it
// cannot be hoisted out of the persistent task loop, which would keep them
// live across every task body and exhaust the register file.
__device__ __forceinline__ int tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

// streaming (non-temporal) loads for data read once per step
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u4v v = __builtin_nontemporal_load((const u4v*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt2(const uint2* p) {
  const u2v v = __builtin_nontemporal_load((const u2v*)p);
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// dot of 8 bf16 weights (one 16-byte chunk) with 8 floats
__device__ __forceinline__ float dot8(const uint4 w, const float* u, float s) {
  s = fmaf(bf_lo(w.x), u[0], s);
  s = fmaf(bf_hi(w.x), u[1], s);
  s = fmaf(bf_lo(w.y), u[2], s);
  s = fmaf(bf_hi(w.y), u[3], s);
  s = fmaf(bf_lo(w.z), u[4], s);
  s = fmaf(bf_hi(w.z), u[5], s);
  s = fmaf(bf_lo(w.w), u[6], s);
  s = fmaf(bf_hi(w.w), u[7], s);
  return s;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each row of 16 lanes; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
// Sum over aligned groups of `width` (32 or 64) lanes; every lane gets its group's sum.
__device__ __forceinline__ float group_sum(float v, int width) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, 64);
  if (width == 64) v += __shfl_xor(v, 32, 64);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ------------------------------------------------------------------ tagged words

__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t* p, float v, uint32_t epoch) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t epoch) { return (uint32_t)(w >> 32) == epoch; }
__device__ __forceinline__ float tag_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Record a device failure: the first one wins the code word.
__device__ __forceinline__ void raise_status(const KArgs& a, uint32_t code, uint32_t w1, uint32_t w2,
                                             uint32_t w3) {
  if (atomicCAS(a.status, 0u, code) == 0u) {
    __hip_atomic_store(a.status + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + 2, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + 3, w3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
__device__ __forceinline__ bool aborted(const KArgs& a) {
  return __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Spin until the word at p carries the current epoch; returns its value.
// A deadline (from t0) or another workgroup's failure sets *fail.
__device__ __forceinline__ float get_tagged(const KArgs& a, const uint64_t* p, uint64_t t0,
                                            uint32_t task, bool* fail) {
  uint64_t w = ld_tagged(p);
  if (tag_is(w, a.epoch)) return tag_value(w);
  uint32_t it = 0;
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    w = ld_tagged(p);
    if (tag_is(w, a.epoch)) return tag_value(w);
    if ((++it & 63u) == 0u) {
      if (aborted(a)) { *fail = true; return 0.f; }
      if (now() - t0 > a.timeout_ticks) {
        raise_status(a, DS_TIMEOUT, task, (uint32_t)(p - a.x), (uint32_t)(w >> 32));
        *fail = true;
        return 0.f;
      }
    }
  }
}

// Read up to MAXW tagged words of this thread, word k at addr(k) (nullptr:
// none), into out[k]. All loads are in flight together; while some words are
// stale the thread spins on its first stale word alone (one load per round)
// and then re-reads the stale set as one batch, so a consumer that starts
// early adds little traffic and one that starts late pays one round trip.
// Returns false on deadline or another workgroup's failure.
template <int MAXW, class Addr>
__device__ __forceinline__ bool read_words(const KArgs& a, const Addr& addr, float* out, uint64_t t0,
                                           uint32_t task) {
  const uint32_t ep = a.epoch;
  uint64_t w[MAXW];
#pragma unroll
  for (int k = 0; k < MAXW; ++k) {
    const uint64_t* p = addr(k);
    w[k] = p ? ld_tagged(p) : ((uint64_t)ep << 32);
  }
  uint32_t stale = 0;
#pragma unroll
  for (int k = 0; k < MAXW; ++k) stale |= tag_is(w[k], ep) ? 0u : (1u << k);
  uint32_t it = 0;
  while (stale) {
    // spin on the first stale word
#pragma unroll
    for (int k = 0; k < MAXW; ++k) {
      if (stale & (1u << k)) {
        const uint64_t* p = addr(k);
        while (true) {
          __builtin_amdgcn_s_sleep(1);
          w[k] = ld_tagged(p);
          if (tag_is(w[k], ep)) break;
          if ((++it & 63u) == 0u) {
            if (aborted(a)) return false;
            if (now() - t0 > a.timeout_ticks) {
              raise_status(a, DS_TIMEOUT, task, (uint32_t)(p - a.x), (uint32_t)(w[k] >> 32));
              return false;
            }
          }
        }
        stale &= ~(1u << k);
        break;
      }
    }
    // then re-read the rest of the stale set together
#pragma unroll
    for (int k = 0; k < MAXW; ++k)
      if (stale & (1u << k)) w[k] = ld_tagged(addr(k));
#pragma unroll
    for (int k = 0; k < MAXW; ++k)
      if ((stale & (1u << k)) && tag_is(w[k], ep)) stale &= ~(1u << k);
  }
#pragma unroll
  for (int k = 0; k < MAXW; ++k) out[k] = tag_value(w[k]);
  return true;
}

}  // namespace dev
}  // namespace mk
