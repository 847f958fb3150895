// Device helpers of the megakernel: bf16 unpacking, wave reductions,
// dependency waits and signals on device-memory counters.
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
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// dot of 8 bf16 weights (one 16-byte chunk) with 8 floats
__device__ __forceinline__ float dot8(const uint4 w, const float* u) {
  float s = bf_lo(w.x) * u[0];
  s = fmaf(bf_hi(w.x), u[1], s);
  s = fmaf(bf_lo(w.y), u[2], s);
  s = fmaf(bf_hi(w.y), u[3], s);
  s = fmaf(bf_lo(w.z), u[4], s);
  s = fmaf(bf_hi(w.z), u[5], s);
  s = fmaf(bf_lo(w.w), u[6], s);
  s = fmaf(bf_hi(w.w), u[7], s);
  return s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// sum over aligned groups of `width` lanes (power of two <= 64)
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Record a device failure: the first one wins the code word.
__device__ __forceinline__ void raise_status(const KArgs& a, uint32_t code, uint32_t w1, uint32_t w2,
                                             uint32_t w3) {
  if (atomicCAS(a.status, 0u, code) == 0u) {
    __hip_atomic_store(a.status + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + 2, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + 3, w3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until counter ci reaches epoch * cnt. Wave 0 spins with relaxed
// device-scope loads and then takes an acquire fence; the other waves wait
// at the barrier, so loads they issued before the wait (weights, old KV)
// stay in flight. Returns false (uniformly) if the step was aborted: this
// wait passed its deadline, or another workgroup recorded a failure.
__device__ __forceinline__ bool wg_wait(const KArgs& a, uint16_t ci, uint16_t cnt, uint32_t task,
                                        int* sflag, uint64_t* tw) {
  if (ci == NO_CTR) return true;
  const uint32_t target = a.epoch * (uint32_t)cnt;
  if (threadIdx.x < 64) {
    if (a.trace && threadIdx.x == 0) tw[0] = __builtin_amdgcn_s_memrealtime();
    const uint32_t* c = a.ctr + (size_t)ci * CTR_STRIDE;
    int ok = 1;
    uint32_t v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v < target) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      uint32_t it = 0;
      while (true) {
        __builtin_amdgcn_s_sleep(1);
        v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v >= target) break;
        if ((++it & 31u) == 0u) {
          if (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
            ok = 0;
            break;
          }
          if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout_ticks) {
            if (threadIdx.x == 0) raise_status(a, DS_TIMEOUT, task, ci, v);
            ok = 0;
            break;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    wait_vm();
    if (threadIdx.x == 0) {
      *sflag = ok;
      if (a.trace) tw[1] = __builtin_amdgcn_s_memrealtime();
    }
  }
  __syncthreads();
  return *sflag != 0;
}

// Publish this task's stores and increment counter ci. Every wave waits for
// its own stores to reach L2 before the barrier; thread 0's agent-scope
// release then writes the L2 back, so consumers on other XCDs (each XCD has
// its own L2) see the whole workgroup's results after their acquire.
__device__ __forceinline__ void wg_signal(const KArgs& a, uint16_t ci) {
  wait_vm();
  __syncthreads();
  if (ci != NO_CTR && threadIdx.x == 0) {
    __hip_atomic_fetch_add(a.ctr + (size_t)ci * CTR_STRIDE, 1u, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace dev
}  // namespace mk
