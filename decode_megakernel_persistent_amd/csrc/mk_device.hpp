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

// The kernel argument block as seen by the task bodies: read in place from
// the kernel-argument segment (constant address space) with scalar loads.
// Holding all of its fields in scalar registers for the whole persistent
// loop would exceed the scalar register file and spill.
typedef const __attribute__((address_space(4))) KArgs KAC;

// The thread index read through an opaque move. Values derived from it
// cannot be hoisted out of the persistent task loop, which would keep them
// live across every task body and exhaust the register file.
__device__ __forceinline__ int tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

// Workgroup barrier for LDS traffic only. Waves of a workgroup share data
// through LDS alone (global data between tasks is synchronised by its tags),
// so a wave need only finish its own LDS accesses before the barrier. A full
// __syncthreads() would also wait for every outstanding global load, including
// weight and direct-to-LDS prefetches that are meant to stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// streaming (non-temporal) loads for data read once per step
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u4v v = __builtin_nontemporal_load((const u4v*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt2(const uint2* p) {
  const u2v v = __builtin_nontemporal_load((const u2v*)p);
  return make_uint2(v.x, v.y);
}

// Direct-to-LDS load of 16 bytes per lane: lane i's 16 bytes from g land at
// LDS byte address lds_base + 16 * i (lds_base wave-uniform). Written as
// inline assembly so that the compiler does not treat every later LDS read
// as possibly aliasing the transfer (it would wait for all outstanding
// vector memory operations before each one); the consumer waits for the
// transfer itself (s_waitcnt vmcnt) before reading its destination.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds_base) : "memory");
}
// Direct-to-LDS load of 4 bytes per lane: lane i's word lands at LDS byte
// address lds_base + 4 * i (lds_base wave-uniform); same waiting rule.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
// 2^x with one v_exp_f32 (about 1 ulp; results below 2^-126 flush to 0,
// 2^-inf = 0): for softmax weights, whose scores are kept in log2 units
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E_F = 1.44269504088896341f;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f2v_t __attribute__((ext_vector_type(2)));
// Two fp32 values to packed bf16 bits (x in bits 0..15, y in 16..31), round
// to nearest even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  const f2v_t v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// fp32 -> bf16 bits, round to nearest even
__device__ __forceinline__ uint32_t f2bf(float f) { return pk_bf16(f, 0.f) & 0xFFFFu; }
// hi/lo bf16 split of a pair: hi = bf16(x) | bf16(y) << 16, lo likewise of
// the residuals x - hi, y - hi (each residual is exact in fp32)
__device__ __forceinline__ void split2(float x, float y, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(x, y);
  lo = pk_bf16(x - bf_lo(hi), y - bf_hi(hi));
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Dot of 8 bf16 weights (one 16-byte chunk) with 8 activations given as a
// hi/lo bf16 split (uh = bf16(u), ul = bf16(u - uh), two per 32-bit word in
// element order): each bf16 x bf16 product is exact in fp32 and u - uh - ul is
// below 2^-18 |u|, so this equals an fp32 dot to within fp32 accumulation.
__device__ __forceinline__ float dot8h(const uint4 w, const uint4 uh, const uint4 ul, float s) {
#define MK_DOT2(a, b) s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), s, false)
  MK_DOT2(w.x, uh.x); MK_DOT2(w.x, ul.x);
  MK_DOT2(w.y, uh.y); MK_DOT2(w.y, ul.y);
  MK_DOT2(w.z, uh.z); MK_DOT2(w.z, ul.z);
  MK_DOT2(w.w, uh.w); MK_DOT2(w.w, ul.w);
#undef MK_DOT2
  return s;
}

// hi/lo bf16 split of 8 floats: words (hi of u[2j] | hi of u[2j+1] << 16), then lo.
__device__ __forceinline__ void split8(const float* u, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split2(u[2 * e], u[2 * e + 1], h[e], l[e]);
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
// Sum over each row of 16 lanes; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
// Sum over aligned groups of TC (32 or 64) lanes, all in DPP (no LDS
// crossbar): the group's sum is valid in its last lane (tc == TC - 1).
template <int TC>
__device__ __forceinline__ float group_sum_last(float v) {
  v = row16_sum(v);
  v += dpp<0x142, 0xA>(v);                    // row_bcast:15 into rows 1 and 3
  if (TC == 64) v += dpp<0x143, 0xC>(v);      // row_bcast:31 into rows 2 and 3
  return v;
}
// Sum over the wave, returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  const float s = group_sum_last<64>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 63));
}
// Maximum over the wave, returned to every lane (DPP, no LDS).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  // rows not written by a broadcast keep their own value: fmax(v, 0) must not
  // see the zero that update_dpp supplies for masked rows, so those rows
  // take the max with themselves instead
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Cross-lane pair operations without the LDS crossbar: v (op) v[lane ^ 8]
// (DPP row rotate by 8 within each row of 16 lanes), v (op) v[lane ^ 16] and
// v (op) v[lane ^ 32] (the gfx950 permlane swaps). Each lane of a pair gets
// the same result.
__device__ __forceinline__ float xor8_sum(float v) { return v + dpp<0x128>(v); }
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

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

// Two neighbouring tagged words (byte offset off, a multiple of 16, in a
// buffer of nbytes at base) read as two 8-byte loads, both in flight
// together, each with the same coherence as ld_tagged (sc1: this XCD's L2 is
// bypassed). Each load is the very instruction that the AMDGPU backend emits
// for a relaxed agent-scope 64-bit atomic load (LLVM "User Guide for AMDGPU
// Backend", memory model code sequences for GFX942, which gfx950 follows:
// load atomic monotonic, agent scope = buffer/global load with sc1), so each
// word arrives whole, as its single 8-byte store wrote it, and its tag
// vouches for its own value. A 16-byte load of the pair would not be an
// atomic access in that model: the scheduling barrier keeps the compiler
// from merging the two loads into one (a CPU test checks the built code
// object for it). The buffer resource makes offsets at or past nbytes read
// zeros (a stale tag), never another allocation. .x/.y = word 0 (value,
// tag), .z/.w = word 1.
typedef __amdgpu_buffer_rsrc_t tag_rsrc;
__device__ __forceinline__ tag_rsrc tagged_rsrc(const uint64_t* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)nbytes, 0x00020000);
}
typedef unsigned int tag_u2 __attribute__((ext_vector_type(2)));
// A caller that re-reads a word in a loop puts a compiler memory barrier
// (tagged_reload_fence) between the reads, so that they are not merged.
__device__ __forceinline__ uint4 ld_tagged2(tag_rsrc r, uint32_t off) {
  const tag_u2 w0 = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16);  // cache policy 16: sc1
  __builtin_amdgcn_sched_barrier(0);
  const tag_u2 w1 = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8u, 0, 16);
  return make_uint4(w0.x, w0.y, w1.x, w1.y);
}
__device__ __forceinline__ void tagged_reload_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ bool tag2_is(const uint4& v, uint32_t epoch) { return v.y == epoch && v.w == epoch; }
__device__ __forceinline__ float tag_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Record a device failure: the first one wins the code word.
__device__ __forceinline__ void raise_status(KAC& a, uint32_t code, uint32_t w1, uint32_t w2,
                                             uint32_t w3) {
  if (atomicCAS(a.status, 0u, code) == 0u) {
    __hip_atomic_store(a.status + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + 2, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + 3, w3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
__device__ __forceinline__ bool aborted(KAC& a) {
  return __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Spin until the word at p carries the current epoch; returns its value.
// A deadline (from t0) or another workgroup's failure sets *fail.
__device__ __forceinline__ float get_tagged(KAC& a, const uint64_t* p, uint64_t t0,
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
// stale the thread re-reads the stale set (again all in flight) after a short
// sleep, so a word is seen within one round trip of its store landing.
// Returns false on deadline or another workgroup's failure.
template <int MAXW, class Addr>
__device__ __forceinline__ bool read_words(KAC& a, const Addr& addr, float* out, uint64_t t0,
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
    // re-read the whole stale set each round, all loads in flight together
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int k = 0; k < MAXW; ++k)
      if (stale & (1u << k)) w[k] = ld_tagged(addr(k));
#pragma unroll
    for (int k = 0; k < MAXW; ++k)
      if ((stale & (1u << k)) && tag_is(w[k], ep)) stale &= ~(1u << k);
    if (stale && (++it & 31u) == 0u) {
      if (aborted(a)) return false;
      if (now() - t0 > a.timeout_ticks) {
        const int k = __builtin_ctz(stale);
        raise_status(a, DS_TIMEOUT, task, (uint32_t)k, 0xFFFFFFFFu);
        return false;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < MAXW; ++k) out[k] = tag_value(w[k]);
  return true;
}

}  // namespace dev
}  // namespace mk
