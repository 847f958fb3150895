// The persistent decode megakernel for gfx950 and its launch.
//
// One workgroup of 512 threads per compute unit walks its own task list
// (megakernel page, "What is a Megakernel?": one resident block per
// processor, work read from a task list in global memory, tasks that wait
// for exactly the producers they read). Every task first issues the loads
// that depend on no other task (weights, KV pages of earlier steps) into
// registers, then waits for its inputs, then computes and publishes.
//
// Synchronisation. Activations pass between tasks as tagged words (epoch in
// the high half, fp32 bits in the low half) written with device-coherent
// stores; a consumer spins on the words themselves until they carry the
// step's epoch. On MI355X each XCD has its own L2, and a counter handoff
// that releases with an L2 writeback and acquires with an L2 invalidate costs
// several microseconds per dependency stage; a tagged word needs neither,
// because the value and its completion mark travel in one coherent access.
// Each task also adds the number of outputs it produced to its completion
// counter (spread over 8 lines), so that a finished step leaves every counter
// at steps x the outputs of its class.
//
// Task bodies:
//  - batch 1: projections (QKV, O, router, expert gate/up, expert down, LM
//    head) are GEMVs: each lane group of 64 (or 32) lanes holds whole rows as
//    16-byte bf16 chunks, accumulates in fp32 and reduces with DPP row
//    operations; RMSNorm is recomputed by every consumer tile from the
//    gathered vector; RoPE + KV append, residual adds, SwiGLU, the weighted
//    expert combine and the local argmax are epilogues;
//  - batches of 2 .. 32 sequences: the same projections as MFMA 16x16x32
//    bf16 tiles (see the batch tasks below);
//  - paged attention splits use MFMA 16x16x32 bf16 tiles on 16-token pages
//    (queries and probabilities carried as bf16 hi + lo pairs), an online
//    softmax across pages and a log-sum-exp merge across waves;
//  - the split combine is a log-sum-exp merge in fixed split order.
// Consumers read neighbouring tagged words in pairs: two 8-byte loads in
// flight together, each a whole tagged word.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "mk.h"
#include "mk_device.hpp"
#include "mk_internal.hpp"
#include "mk_plan.hpp"

namespace mk {
namespace dev {

constexpr int LDS_VEC = dev_lds_vec();

constexpr int STAGE_CHUNKS = 12;  // 1 KB wave chunks per wave in the shared area (96 KB)
constexpr int DOWN_CHUNKS = 12;   // 16-byte chunks per lane of an expert task's down-projection tile

// Attention: register page buffers per wave, and the page ids of a split
// that are read ahead with its staged pages.
constexpr int ATT_NBUF = 4;
constexpr int ATT_IDS = NWAVE * ATT_NBUF;

struct Smem {
  float vec[LDS_VEC];  // gathered input vector(s), normalised in place
  union {
    uint4 stage[NWAVE * STAGE_CHUNKS * 64];  // batch tasks: staged operands
    float att[NWAVE * STAGE_CHUNKS * 256];   // attention: per-wave partials; combine: split words
  };
  alignas(16) float out[2048];     // per-row dot products
  float res[2048];     // residual rows
  float red[64];       // block reductions
  float route_w[16];
  alignas(16) float route_wn[16];  // routing weights as applied (renormalised when the model says so)
  int route_ids[16];
  int fail;
  int kv_ti;                 // task index of the attention split whose pages are staged (-1: none)
  int kv_ok[STAGE_PAGES];    // staged page k of the split is valid
  int kv_ids[ATT_IDS + 1];   // its first ATT_IDS page ids, then the sequence's position
  uint32_t qnext;      // attention queue: the split this workgroup takes next
  int tok;             // sampling: the drawn token
  uint64_t tw[4];      // trace: (begin, end) of the routing wait and of the data wait
  uint64_t mk[TRACE_MARKS];  // trace: body-specific marks
};

struct Ctx {
  KAC& a;
  Smem& s;
  uint64_t t0;
  uint32_t ti;
};

// Trace mark i of the current task (no-op without a trace buffer).
__device__ __forceinline__ void mark(Ctx& c, int i) {
  if (c.a.trace && tid() == 0) c.s.mk[i] = now();
}

// Order-preserving 64-bit rank key of router logit v of expert e: a larger
// logit ranks first, and on equal logits the lower index. (The softmax is
// monotone, so ranking logits ranks the probabilities.)
__device__ __forceinline__ uint64_t logit_key(float v, int e) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFF - e);
}

// Byte offset of a tagged word in the workspace.
__device__ __forceinline__ uint32_t ws_off(const KAC& a, const uint64_t* p) {
  return (uint32_t)((const char*)p - (const char*)a.ws);
}

// Read MAXP pairs of neighbouring tagged words of this thread (pair k at
// workspace byte offset off(k), a multiple of 16, or NO_PAIR) into out[2k],
// out[2k + 1], two 8-byte loads per pair (ld_tagged2), re-reading stale pairs like
// read_words. Returns false on deadline or another workgroup's failure.
constexpr uint32_t NO_PAIR = 0xFFFFFFFFu;
template <int MAXP, class Off>
__device__ __forceinline__ bool read_pairs(KAC& a, const Off& off, float* out, uint64_t t0, uint32_t task) {
  const tag_rsrc r = tagged_rsrc(a.ws, a.ws_bytes);
  const uint32_t ep = a.epoch;
  uint4 w[MAXP];
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    const uint32_t o = off(k);
    w[k] = o != NO_PAIR ? ld_tagged2(r, o) : make_uint4(0u, ep, 0u, ep);
  }
  uint32_t stale = 0;
#pragma unroll
  for (int k = 0; k < MAXP; ++k) stale |= tag2_is(w[k], ep) ? 0u : (1u << k);
  uint32_t it = 0;
  while (stale) {
    __builtin_amdgcn_s_sleep(2);
    tagged_reload_fence();
#pragma unroll
    for (int k = 0; k < MAXP; ++k)
      if (stale & (1u << k)) w[k] = ld_tagged2(r, off(k));
#pragma unroll
    for (int k = 0; k < MAXP; ++k)
      if ((stale & (1u << k)) && tag2_is(w[k], ep)) stale &= ~(1u << k);
    if (stale && (++it & 31u) == 0u) {
      if (aborted(a)) return false;
      if (now() - t0 > a.timeout_ticks) {
        raise_status(a, DS_TIMEOUT, task, (uint32_t)__builtin_ctz(stale), 0xFFFFFFFDu);
        return false;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    out[2 * k] = __uint_as_float(w[k].x);
    out[2 * k + 1] = __uint_as_float(w[k].z);
  }
  return true;
}

// Gather tagged words into LDS: dst[i] = value of word i for i < n, where
// word i sits at src1 + i for i < n1 and at src2 + (i - n1) after that,
// read as pairs (2j, 2j + 1) with ld_tagged2: n1 and n are even
// and both sources start at an even workspace word (the planner lays out
// every buffer so). MAXW words per thread per batch. which: 0 = routing
// wait, 1 = data wait (trace slots), -1 = untraced. With nsq > 0 the sum of
// squares of words 0 .. nsq-1 is formed on the way (each thread over its
// words in order, then over the wave) and wave w's part is left in s.red[w]
// for norm_pack. With keys, the words of src2 are router logits: their rank
// keys go to keys[] and the per-wave maxima to s.red[NWAVE + w]. Uniform
// result.
template <int MAXW>
__device__ __forceinline__ bool gather2(Ctx& c, const uint64_t* src1, int n1, const uint64_t* src2, int n,
                                        float* dst, int which, int nsq = 0, uint64_t* keys = nullptr) {
  KAC& a = c.a;
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which] = now();
  bool ok = true;
  float ss = 0.f, mx = NEG_INF;
  constexpr int MAXP = (MAXW + 1) / 2;
  const uint32_t o1 = ws_off(a, src1), o2 = ws_off(a, src2);
  for (int base = 0; base < n && ok; base += 2 * MAXP * NT) {
    const int t = tid();
    float v[2 * MAXP];
    ok = read_pairs<MAXP>(a, [&](int k) -> uint32_t {
      const int i = base + 2 * (t + k * NT);
      return i < n1 ? o1 + 8u * i : (i < n ? o2 + 8u * (i - n1) : NO_PAIR);
    }, v, c.t0, c.ti);
    if (ok) {
#pragma unroll
      for (int k = 0; k < MAXP; ++k) {
        const int i = base + 2 * (t + k * NT);
        if (i < n) *(float2*)(dst + i) = make_float2(v[2 * k], v[2 * k + 1]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if (i + e < nsq) ss = fmaf(v[2 * k + e], v[2 * k + e], ss);
          if (keys && i + e >= n1 && i + e < n) {
            keys[i + e - n1] = logit_key(v[2 * k + e], i + e - n1);
            mx = fmaxf(mx, v[2 * k + e]);
          }
        }
      }
    }
  }
  if (nsq > 0) {
    ss = wave_sum(ss);
    if ((tid() & 63) == 0) c.s.red[tid() >> 6] = ss;
  }
  if (keys) {  // the second source holds router logits: rank keys and per-wave maxima
    const int pad = ((n - n1 + 31) & ~31) - (n - n1);
    if (tid() < pad) keys[n - n1 + tid()] = 0ull;
    mx = wave_max_dpp(mx);
    if ((tid() & 63) == 0) c.s.red[NWAVE + (tid() >> 6)] = mx;
  }
  if (!ok) c.s.fail = 1;
  lds_barrier();
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which + 1] = now();
  return c.s.fail == 0;
}
template <int MAXW>
__device__ __forceinline__ bool gather(Ctx& c, const uint64_t* src, int n, float* dst, int which, int nsq = 0) {
  return gather2<MAXW>(c, src, n, src, n, dst, which, nsq);
}

// Gather n tagged words (n even, src at an even workspace word) into LDS
// already in split form (see pack_lds): the pair (2j, 2j + 1) arrives in one
// read (ld_tagged2), and its bf16 hi and lo parts land in chunk 2j / 8, so no
// separate conversion pass or barrier follows. Uniform result.
template <int MAXW>
__device__ __forceinline__ bool gather_split(Ctx& c, const uint64_t* src, int n, float* dst, int which) {
  KAC& a = c.a;
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which] = now();
  uint32_t* dw = (uint32_t*)dst;
  bool ok = true;
  constexpr int MAXP = (MAXW + 1) / 2;
  const uint32_t o = ws_off(a, src);
  for (int base = 0; base < n && ok; base += 2 * MAXP * NT) {
    const int t = tid();
    float v[2 * MAXP];
    ok = read_pairs<MAXP>(a, [&](int k) -> uint32_t {
      const int i = base + 2 * (t + k * NT);
      return i < n ? o + 8u * i : NO_PAIR;
    }, v, c.t0, c.ti);
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const int i = base + 2 * (t + k * NT);
      uint32_t hw, lw;
      split2(v[2 * k], v[2 * k + 1], hw, lw);
      if (ok && i < n) {
        const int ch = i >> 3, e = i & 7;
        dw[8 * ch + (e >> 1)] = hw;
        dw[8 * ch + 4 + (e >> 1)] = lw;
      }
    }
  }
  if (!ok) c.s.fail = 1;
  lds_barrier();
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which + 1] = now();
  return c.s.fail == 0;
}

struct IdentIdx {
  __device__ __forceinline__ int operator()(int i) const { return i; }
};

// Gather n tagged words, word i at addr(i), into dst[di(i)] (LDS); uniform result.
template <int MAXW, class Addr, class DstIdx = IdentIdx>
__device__ __forceinline__ bool gather_fn(Ctx& c, int n, const Addr& addr, float* dst, int which,
                                          const DstIdx& di = DstIdx()) {
  KAC& a = c.a;
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which] = now();
  bool ok = true;
  for (int base = 0; base < n && ok; base += MAXW * NT) {
    const int t = tid();
    float v[MAXW];
    ok = read_words<MAXW>(a, [&](int k) -> const uint64_t* {
      const int i = base + t + k * NT;
      return i < n ? addr(i) : nullptr;
    }, v, c.t0, c.ti);
    if (ok) {
#pragma unroll
      for (int k = 0; k < MAXW; ++k) {
        const int i = base + t + k * NT;
        if (i < n) dst[di(i)] = v[k];
      }
    }
  }
  if (!ok) c.s.fail = 1;
  lds_barrier();
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which + 1] = now();
  return c.s.fail == 0;
}

// gather_fn reading word pairs (i, i + 1), i even, with one ld_tagged2:
// for the caller, n is even and, for every even i, addr(i) (nullptr: none) is
// a word at an even workspace word offset followed by word i + 1, and
// di(i + 1) = di(i) + 1 with di(i) even. Uniform result.
template <int MAXW, class Addr, class DstIdx = IdentIdx>
__device__ __forceinline__ bool gather_fn_pairs(Ctx& c, int n, const Addr& addr, float* dst, int which,
                                                const DstIdx& di = DstIdx()) {
  KAC& a = c.a;
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which] = now();
  constexpr int MAXP = (MAXW + 1) / 2;
  bool ok = true;
  for (int base = 0; base < n && ok; base += 2 * MAXP * NT) {
    const int t = tid();
    float v[2 * MAXP];
    ok = read_pairs<MAXP>(a, [&](int k) -> uint32_t {
      const int i = base + 2 * (t + k * NT);
      const uint64_t* p = i < n ? addr(i) : nullptr;
      return p ? ws_off(a, p) : NO_PAIR;
    }, v, c.t0, c.ti);
    if (ok) {
#pragma unroll
      for (int k = 0; k < MAXP; ++k) {
        const int i = base + 2 * (t + k * NT);
        if (i < n) *(float2*)(dst + di(i)) = make_float2(v[2 * k], v[2 * k + 1]);
      }
    }
  }
  if (!ok) c.s.fail = 1;
  lds_barrier();
  if (which >= 0 && a.trace && tid() == 0) c.s.tw[2 * which + 1] = now();
  return c.s.fail == 0;
}

// Norm gains of chunk tid (elements 8*tid .. 8*tid+7) of a vector of K <=
// 8*NT elements, loaded ahead of a task's wait.
struct Gains {
  uint4 g;
  __device__ __forceinline__ void load(const uint16_t* src, int K) {
    g = tid() < K / 8 ? *(const uint4*)(src + 8 * tid()) : make_uint4(0, 0, 0, 0);
  }
};

// A GEMV input vector in LDS is stored in split form: chunk c (elements
// 8c .. 8c+7) holds 4 words of hi bf16 pairs then 4 words of lo bf16 pairs
// (split8) in place of its 8 floats. pack_lds converts fp32 v[0..K) in place;
// rmsnorm_pack first normalises: v = v / sqrt(mean(v^2) + eps) * g (fixed
// summation order: per chunk, then waves in order).
__device__ __forceinline__ void pack_lds(Ctx& c, float* v, int K) {
  for (int ch = tid(); ch < K / 8; ch += NT) {
    float x[8];
    *(float4*)x = *(const float4*)(v + 8 * ch);
    *(float4*)(x + 4) = *(const float4*)(v + 8 * ch + 4);
    uint4 hi, lo;
    split8(x, hi, lo);
    *(uint4*)(v + 8 * ch) = hi;
    *(uint4*)(v + 8 * ch + 4) = lo;
  }
  lds_barrier();
}

// The second half of rmsnorm_pack, for a vector whose sum of squares the
// gather already left in s.red (per wave): scale by the gains and pack.
__device__ __forceinline__ void norm_pack(Ctx& c, float* v, int K, const Gains& gn) {
  const int t = tid();
  float x[8];
  if (t < K / 8) {
    *(float4*)x = *(const float4*)(v + 8 * t);
    *(float4*)(x + 4) = *(const float4*)(v + 8 * t + 4);
  }
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) tot += c.s.red[w];
  const float rs = 1.0f / sqrtf(tot / (float)K + c.a.eps);
  if (t < K / 8) {
    const uint32_t gw[4] = {gn.g.x, gn.g.y, gn.g.z, gn.g.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * rs * ((e & 1) ? bf_hi(gw[e >> 1]) : bf_lo(gw[e >> 1]));
    uint4 hi, lo;
    split8(x, hi, lo);
    *(uint4*)(v + 8 * t) = hi;
    *(uint4*)(v + 8 * t + 4) = lo;
  }
  lds_barrier();
}

__device__ __forceinline__ void rmsnorm_pack(Ctx& c, float* v, int K, const Gains& gn) {
  const int t = tid();
  float x[8];
  float ss = 0.f;
  if (t < K / 8) {
    *(float4*)x = *(const float4*)(v + 8 * t);
    *(float4*)(x + 4) = *(const float4*)(v + 8 * t + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) c.s.red[t >> 6] = ss;
  lds_barrier();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) tot += c.s.red[w];
  const float rs = 1.0f / sqrtf(tot / (float)K + c.a.eps);
  if (t < K / 8) {
    const uint32_t gw[4] = {gn.g.x, gn.g.y, gn.g.z, gn.g.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * rs * ((e & 1) ? bf_hi(gw[e >> 1]) : bf_lo(gw[e >> 1]));
    uint4 hi, lo;
    split8(x, hi, lo);
    *(uint4*)(v + 8 * t) = hi;
    *(uint4*)(v + 8 * t + 4) = lo;
  }
  lds_barrier();
}

// ------------------------------------------------------------------ GEMV tiles

// A tile of R rows of K = TC*CPL*8 bf16 elements held in registers: lane
// group lg (TC lanes) holds rows lg, lg + G, ... (G lane groups), each as
// CPL 16-byte chunks per lane (chunk index tc + c*TC). Loads are issued by
// issue() before the task waits; dots() reduces each row against the LDS
// vector and writes out[row].
template <int CPL, int RPW, int TC>
struct Tile {
  static constexpr int G = NT / TC;
  uint4 w[RPW][CPL];
  int nr, lg, tc;

  template <class RowPtr>
  __device__ __forceinline__ void issue(int R, const RowPtr& rowptr) {
    lg = tid() / TC;
    tc = tid() % TC;
    nr = lg < R ? (R - lg + G - 1) / G : 0;
    if (TC == 64) nr = __builtin_amdgcn_readfirstlane(nr);  // one lane group per wave
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      if (r < nr) {
        const uint4* p = rowptr(lg + r * G);
#pragma unroll
        for (int c = 0; c < CPL; ++c) w[r][c] = ld_nt(p + tc + c * TC);
      }
  }
  // u: split-form input vector (see pack_lds)
  __device__ __forceinline__ void dots(const float* u, float* out) {
    float acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint4* up = (const uint4*)(u + (tc + c * TC) * 8);
      const uint4 uh = up[0], ul = up[1];
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        if (r < nr) acc[r] = dot8h(w[r][c], uh, ul, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      if (r < nr) {
        const float s = group_sum_last<TC>(acc[r]);
        if (tc == TC - 1) out[lg + r * G] = s;
      }
  }
};

// Token id of sequence b, checked against the vocabulary.
__device__ __forceinline__ int token_row(KAC& a, int b) {
  int tok = a.tok_in[b];
  if (tok < 0 || tok >= a.V) {  // an id outside the vocabulary reads row 0 and is reported
    if (tid() == 0) raise_status(a, DS_BOUNDS, 0xFFFFFFFFu, (uint32_t)tok, 0u);
    tok = 0;
  }
  return tok;
}

// Running argmax with ties to the lower index, without branches (a
// short-circuit condition here compiles to divergent branches per element).
__device__ __forceinline__ void argmax_merge(float v, int i, float& bv, int& bi) {
  const bool take = (int)(v > bv) | ((int)(v == bv) & (int)(i < bi));
  bv = take ? v : bv;
  bi = take ? i : bi;
}

// Hidden state entering layer l of sequence b into LDS dst: the embedding
// row for l = 0 (bf16, no wait), else the tagged output of layer l - 1.
__device__ __forceinline__ bool layer_input(Ctx& c, int l, int b, float* dst) {
  KAC& a = c.a;
  if (l == 0) {
    const uint16_t* e = a.embed + (size_t)token_row(a, b) * a.H;
    float ss = 0.f;
    for (int i = tid(); i < a.H; i += NT) {
      const float v = bf2f(e[i]);
      dst[i] = v;
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((tid() & 63) == 0) c.s.red[tid() >> 6] = ss;
    lds_barrier();
    return true;
  }
  return gather<4>(c, a.x + (size_t)(l - 1) * a.s_x + (size_t)b * a.H, a.H, dst, 1, a.H);
}

// Residual value of row r entering layer l (read once the layer's inputs are known complete).
__device__ __forceinline__ float resid(Ctx& c, int l, int b, int r, bool* fail) {
  KAC& a = c.a;
  if (l == 0) return bf2f(a.embed[(size_t)token_row(a, b) * a.H + r]);
  return get_tagged(a, a.x + (size_t)(l - 1) * a.s_x + (size_t)b * a.H + r, c.t0, c.ti, fail);
}

// ------------------------------------------------------------------ routing

// softmax over the E router logits in r (LDS), then top-k with ties to the
// lower index: the rank of expert e is the number of experts with a larger
// probability, or an equal one and a lower index, so the k selected experts
// land in rank order without a serial selection loop. The result is in
// s.route_ids / s.route_w (selected probabilities, not yet renormalised: see
// route_div) after the final barrier.
__device__ __forceinline__ void route(Ctx& c, const float* r) {
  KAC& a = c.a;
  Smem& s = c.s;
  const int t = tid(), E = a.E;
  const int E32 = (E + 31) & ~31;
  uint64_t* keys = (uint64_t*)(s.out + 1024);  // [E32] (padding keys 0 rank below all)
  float* prob = s.out + 1536;                  // [E]
  int* partial = (int*)(s.out + 512);          // [parts][E32] (parts * E32 <= 512)
  // softmax in wave 0 (E <= 256: four logits per lane), no block reductions
  if (t < 64) {
    float v[4], ex[4];
    float m = NEG_INF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = t + 64 * i;
      v[i] = e < E ? r[e] : NEG_INF;
      m = fmaxf(m, v[i]);
    }
    const float M = wave_max_dpp(m);
    float sl = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ex[i] = t + 64 * i < E ? expf(v[i] - M) : 0.f;
      sl += ex[i];
    }
    const float S = wave_sum(sl);
    // Rank key of an expert: its probability's bits above its inverted index
    // (non-negative floats order as their bit patterns; on equal
    // probabilities the lower index ranks first). Keys are unique.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = t + 64 * i;
      const float pe = ex[i] / S;
      if (e < E) prob[e] = pe;
      if (e < E32) keys[e] = e < E ? ((uint64_t)__float_as_uint(pe) << 32) | (uint32_t)(0xFFFF - e) : 0ull;
    }
  }
  lds_barrier();
  // rank = number of keys ahead; thread t counts part t / E32 of the keys for
  // expert t % E32, then the parts are summed
  const int parts = E32 <= 128 ? 4 : 2;
  const int chunk = E32 / parts;  // a multiple of 8
  {
    const int te = t % E32, part = t / E32;
    if (part < parts) {
      const uint64_t mine = keys[te];
      int cnt = 0;
#pragma unroll 2
      for (int e = part * chunk; e < (part + 1) * chunk; e += 8) {
        uint4 q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = *(const uint4*)(keys + e + 2 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cnt += ((((uint64_t)q[i].y << 32) | q[i].x) > mine) ? 1 : 0;
          cnt += ((((uint64_t)q[i].w << 32) | q[i].z) > mine) ? 1 : 0;
        }
      }
      partial[part * E32 + te] = cnt;
    }
  }
  lds_barrier();
  if (t < E) {
    int rank = 0;
    for (int q = 0; q < parts; ++q) rank += partial[q * E32 + t];
    if (rank < a.K) {
      s.route_ids[rank] = t;
      s.route_w[rank] = prob[t];
    }
  }
  lds_barrier();
}

// Divisor of the routing weights: the sum of the selected probabilities (in
// slot order) when they are renormalised over the selection, else 1.
__device__ __forceinline__ float route_div(KAC& a, const Smem& s) {
  if (!a.norm_topk) return 1.f;
  float w = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) w += i < a.K ? s.route_w[i] : 0.f;
  return w;
}

// ------------------------------------------------------------------ tasks

template <int CPL, int TC, int D>
__device__ __forceinline__ bool task_qkv(Ctx& c, const Task& t) {
  constexpr int RPW = GEMV_REG_CHUNKS / CPL < GEMV_RPW_MAX ? GEMV_REG_CHUNKS / CPL : GEMV_RPW_MAX;
  KAC& a = c.a;
  const int l = t.layer, g = t.a0, p0 = t.a1, np = t.a2, nj = 2 * np;
  const int H = a.H;
  const int QR = (a.Hq + 2 * a.Hkv) * D;
  const uint16_t* W = a.wqkv + (size_t)l * QR * H;
  Tile<CPL, RPW, TC> tile;
  tile.issue(nj, [&](int j) {
    int head, i, row;
    qkv_pair(p0 + (j >> 1), g, a.HG, D, a.Hq, a.Hkv, &head, &i, &row);
    return (const uint4*)(W + (size_t)(row + (j & 1) * (D / 2)) * H);
  });
  Gains gn;
  gn.load(a.attn_norm + (size_t)l * H, H);
  // the step's position, its page and rotation: independent of other tasks, loaded ahead
  const int pos = a.seq_lens[0];
  const bool in_bounds = pos >= 0 && pos + 1 <= a.bound && pos < a.n_rope;
  const int pc = in_bounds ? pos : 0;
  const int32_t phys = a.page_table[pc >> 4];
  const int q_me = tid();
  float cs = 1.f, sn = 0.f;
  int head = 0, i = 0, row = 0, sec = 2;
  if (q_me < np) {
    sec = qkv_pair(p0 + q_me, g, a.HG, D, a.Hq, a.Hkv, &head, &i, &row);
    if (sec < 2) {
      cs = a.rope_cos[(size_t)pc * (D / 2) + i];
      sn = a.rope_sin[(size_t)pc * (D / 2) + i];
    }
  }
  if (!layer_input(c, l, 0, c.s.vec)) return false;
  mark(c, 0);
  norm_pack(c, c.s.vec, H, gn);
  mark(c, 1);
  tile.dots(c.s.vec, c.s.out);
  lds_barrier();
  mark(c, 2);
  const bool page_ok = in_bounds && phys >= 0 && phys < a.n_pages;
  if (!page_ok && tid() == 0) raise_status(a, DS_BOUNDS, c.ti, (uint32_t)pos, (uint32_t)phys);
  if (q_me < np) {  // np <= NT: one rotary pair per thread
    const float y0 = c.s.out[2 * q_me], y1 = c.s.out[2 * q_me + 1];
    float r0 = y0, r1 = y1;
    if (sec < 2) {
      r0 = y0 * cs - y1 * sn;
      r1 = y1 * cs + y0 * sn;
    }
    if (sec == 0) {
      uint64_t* qd = a.q + (size_t)l * a.s_q + (size_t)head * D;
      st_tagged(qd + i, r0, a.epoch);
      st_tagged(qd + i + D / 2, r1, a.epoch);
    } else {
      const uint32_t bb = pk_bf16(r0, r1), b0 = bb & 0xFFFFu, b1 = bb >> 16;
      uint64_t* kn = a.kvn + (size_t)l * a.s_kvn + ((size_t)g * 2 + (sec - 1)) * D;
      st_tagged(kn + i, __uint_as_float(b0), a.epoch);
      st_tagged(kn + i + D / 2, __uint_as_float(b1), a.epoch);
      if (page_ok) {
        uint16_t* base = a.pool + (size_t)phys * a.page_stride + (size_t)l * a.layer_stride +
                         (size_t)g * 2 * 16 * D;
        const int slot = pos & 15;
        if (sec == 1) {
          base[kv_k_offset(slot, i)] = (uint16_t)b0;
          base[kv_k_offset(slot, i + D / 2)] = (uint16_t)b1;
        } else {
          base[kv_v_offset(slot, i, D)] = (uint16_t)b0;
          base[kv_v_offset(slot, i + D / 2, D)] = (uint16_t)b1;
        }
      }
    }
  }
  return true;
}

// Staged attention page k of a split (one (page, layer, kv head) block of
// 2 x 16 x D bf16, in pool order) in the shared area. The split's per-wave
// partials overlay the first pages: every wave reads its staged pages into
// registers before the query gather's barrier and writes its partial after
// it.
template <int D>
__device__ __forceinline__ uint4* staged_page(Smem& s, int k) {
  return s.stage + k * (4 * D);
}
static_assert(STAGE_PAGES * 4 * 128 * 16 <= NWAVE * STAGE_CHUNKS * 64 * 16, "staged pages fit the shared area");
static_assert(NWAVE * 8 * 128 * 4 <= NWAVE * STAGE_CHUNKS * 64 * 16, "attention partials fit the shared area");

// Request the first pages of this unit's next attention split ta (task index
// ti_a of this unit's list) into LDS, wave w taking pages w and w + NWAVE
// (the ones it computes first), with direct-to-LDS
// loads: at the start of the unit's expert task, while it waits for the
// routing decision and HBM is otherwise idle, so that the split computes from
// LDS as soon as its queries arrive. The split's own wave w waits for the
// transfer (vmcnt). (Issued after the routing gather instead, the step was
// 2 % slower.)
template <int D>
__device__ __forceinline__ void stage_kv(Ctx& c, const Task& ta, uint32_t ti_a) {
  KAC& a = c.a;
  Smem& s = c.s;
  const int w = tid() >> 6, lane = tid() & 63;
  const int b = ta.a0, g = ta.a1, pg0 = ta.a2, npg = ta.a3, l = ta.layer;
  const int nst = min(npg, STAGE_PAGES);
  int32_t phys[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int k = w + NWAVE * j;
    phys[j] = k < nst ? a.page_table[(size_t)b * a.max_pages + pg0 + k] : -1;
  }
  bool ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int k = w + NWAVE * j;
    ok[j] = k < nst && phys[j] >= 0 && phys[j] < a.n_pages;
    if (ok[j]) {
      const uint4* src = (const uint4*)(a.pool + (size_t)phys[j] * a.page_stride + (size_t)l * a.layer_stride +
                                        (size_t)g * 2 * 16 * D) + lane;
      uint4* dst = staged_page<D>(s, k);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) dma16(src + 64 * i, lds_addr(dst + 64 * i));
    }
  }
  // the ids of the split's first ATT_IDS pages and the position, so that the
  // split issues its page loads without a page-table round trip
  if (w == 0) {
    const int32_t* prow = a.page_table + (size_t)b * a.max_pages + pg0;
    if (lane < min(npg, ATT_IDS)) dma4(prow + lane, lds_addr(s.kv_ids));
    else if (lane == ATT_IDS) dma4(a.seq_lens + b, lds_addr(s.kv_ids));
  }
  if (lane == 0) {
    s.kv_ok[w] = ok[0] ? 1 : 0;
    if (w + NWAVE < STAGE_PAGES) s.kv_ok[w + NWAVE] = ok[1] ? 1 : 0;
  }
  if (tid() == 0) s.kv_ti = (int)ti_a;
}

template <int D>
__device__ __forceinline__ bool task_attn(Ctx& c, const Task& t) {
  constexpr int NK4 = D / 32;   // 16-byte K loads per lane per page
  constexpr int NB = D / 16;    // 16-dim blocks of the PV product
  constexpr int NS = D / 32;    // MFMA k-steps of the QK product (16x16x32)
  KAC& a = c.a;
  Smem& s = c.s;
  const int l = t.layer, b = t.a0, g = t.a1, pg0 = t.a2, npg = t.a3, split = t.aux;
  const int HG = a.HG;
  if ((t.flags & TF_PREFILL) && b > 0) {
    // chunk row b reads pool slots that rows 0 .. b-1 write in this step:
    // wait for those rows' K and V words of this head (each stored after its
    // writer released its pool slots), then acquire
    const int n = b * 2 * D;
    bool ok = true;
    for (int base = 0; base < n && ok; base += NT * 4) {
      float v[4];
      ok = read_words<4>(a, [&](int k) -> const uint64_t* {
        const int i = base + tid() + k * NT;
        if (i >= n) return nullptr;
        const int j = i / (2 * D), e = i - j * 2 * D;
        return a.kvn + (size_t)l * a.s_kvn + ((size_t)j * a.Hkv + g) * 2 * D + e;
      }, v, c.t0, c.ti);
    }
    if (!ok) s.fail = 1;
    lds_barrier();
    if (s.fail) return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  const int lane = tid() & 63, w = tid() >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int32_t* prow = a.page_table + (size_t)b * a.max_pages;
  // Pages stream through a ring of NBUF register buffers per wave (wave w
  // takes the task's pages w, w + NWAVE, ...). The wave's first NBUF page ids
  // are read directly, together with the position; the ids of every page of
  // the task go to an LDS table for the rest, so a refill never waits on a
  // page-table load (the plan maps every page below its bound).
  constexpr int NBUF = ATT_NBUF;
  const int first = pg0 + w;
  // ids and position read ahead by stage_kv (in LDS since the staging task's
  // first wait for its loads), else from memory
  const bool pre = s.kv_ti == (int)c.ti;
  int32_t ph[NBUF];
#pragma unroll
  for (int j = 0; j < NBUF; ++j)
    ph[j] = first + j * NWAVE < pg0 + npg ? (pre ? s.kv_ids[w + j * NWAVE] : prow[first + j * NWAVE]) : -1;
  const int pos = pre ? s.kv_ids[ATT_IDS] : a.seq_lens[b];
  // the id table for refills (pages past each wave's first NBUF)
  const bool refill = npg > NWAVE * NBUF;
  int* pid = (int*)s.res;  // [npg]
  int32_t tbl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) tbl[j] = refill && tid() + j * NT < npg ? prow[pg0 + tid() + j * NT] : -1;
  const int n_tok = min(pos + 1, a.bound);
  const int pg_lim = min(pg0 + npg, (n_tok + 15) >> 4);
  const int cnt = first < pg_lim ? (pg_lim - first + NWAVE - 1) / NWAVE : 0;
  const int cur = pos >> 4, ns = pos & 15;
  const uint16_t* lbase = a.pool + (size_t)l * a.layer_stride + (size_t)g * 2 * 16 * D;
  uint4 kb[NBUF][NK4];
  uint2 vb[NBUF][NB];
  bool bad = false;
  auto load = [&](uint4 (&kk)[NK4], uint2 (&vv)[NB], int pg, int32_t phys) {
    if (phys < 0 || phys >= a.n_pages) {
      bad = true;
#pragma unroll
      for (int i = 0; i < NK4; ++i) kk[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NB; ++i) vv[i] = make_uint2(0, 0);
      return;
    }
    // the page block is stored in operand order (kv_k_offset, kv_v_offset):
    // K chunk i of this lane (dims 32 i + 8 kq .. + 7 of slot r16) and V chunk
    // m (slots 4 kq .. + 3 of dims 32 m + r16 and 32 m + 16 + r16) are the
    // lane's 16 bytes of one contiguous kilobyte
    const uint4* kp = (const uint4*)(lbase + (size_t)phys * a.page_stride) + lane;
#pragma unroll
    for (int i = 0; i < NK4; ++i) kk[i] = ld_nt(kp + 64 * i);
#pragma unroll
    for (int m = 0; m < NB / 2; ++m) {
      const uint4 v = ld_nt(kp + 2 * D + 64 * m);
      vv[2 * m] = make_uint2(v.x, v.y);
      vv[2 * m + 1] = make_uint2(v.z, v.w);
    }
  };
  // this wave's first two pages may have been staged in LDS by an earlier
  // task of this unit (stage_kv): that task waited for loads it issued after
  // the transfer, so the pages have landed
  bool staged[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int k = w + NWAVE * j;
    staged[j] = j < cnt && k < STAGE_PAGES && pre && s.kv_ok[k];
    if (staged[j]) {
      const uint4* sp = staged_page<D>(s, k) + lane;
#pragma unroll
      for (int i = 0; i < NK4; ++i) kb[j][i] = sp[64 * i];
#pragma unroll
      for (int m = 0; m < NB / 2; ++m) {
        const uint4 v = sp[2 * D + 64 * m];
        vb[j][2 * m] = make_uint2(v.x, v.y);
        vb[j][2 * m + 1] = make_uint2(v.z, v.w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NBUF; ++j)
    if (j < cnt && !(j < 2 && staged[j])) load(kb[j], vb[j], first + j * NWAVE, ph[j]);
  if (refill)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (tid() + j * NT < npg) pid[tid() + j * NT] = tbl[j];

  // inputs: the group's queries and the new token's K and V (bf16 bits), one batch
  float* qv = s.vec;                 // [HG][D]
  float* kvnew = s.vec + HG * D;     // [2][D]
  const uint64_t* qsrc = a.q + (size_t)l * a.s_q + ((size_t)b * a.Hq + (size_t)g * HG) * D;
  const uint64_t* ksrc = a.kvn + (size_t)l * a.s_kvn + ((size_t)b * a.Hkv + g) * 2 * D;
  mark(c, 0);
  if (!gather2<3>(c, qsrc, HG * D, ksrc, HG * D + 2 * D, qv, 1)) return false;
  mark(c, 1);

  // query operand: column r16 < 8 carries bf16(q) of head r16, column
  // r16 >= 8 the bf16 residual q - bf16(q) of head r16 - 8
  const int hh = r16 & 7;
  const bool lo_part = r16 >= 8;
  // k-step st (MFMA 16x16x32) covers dims 32 st + 8 kq .. + 7, as K chunk st
  uint4 qop[NS];
  {
    const bool valid = hh < HG;
    const float* qp = qv + (valid ? hh : 0) * D + 8 * kq;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      uint32_t h[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float4 x = valid ? *(const float4*)(qp + 32 * st + 4 * half) : make_float4(0.f, 0.f, 0.f, 0.f);
        uint32_t hw, lw;
        split2(x.x, x.y, hw, lw);
        h[2 * half] = lo_part ? lw : hw;
        split2(x.z, x.w, hw, lw);
        h[2 * half + 1] = lo_part ? lw : hw;
      }
      qop[st] = make_uint4(h[0], h[1], h[2], h[3]);
    }
  }
  mark(c, 4);
  float m_run = NEG_INF, l_run = 0.f;
  v4f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  // scores in log2 units (scale log2 e), so that every softmax weight is one
  // 2^x; the partial maxima published below are in the same units
  const float scale = a.attn_scale * LOG2E_F;
  // the new token's slot of page pg: its K and V come from this step's QKV tasks
  auto patch = [&](uint4 (&kk)[NK4], uint2 (&vv)[NB], int pg) {
    if (pg != cur) return;
    if (r16 == ns) {
#pragma unroll
      for (int i = 0; i < NK4; ++i) {
        const float* kn = kvnew + 8 * kq + 32 * i;
        kk[i] = make_uint4(__float_as_uint(kn[0]) | (__float_as_uint(kn[1]) << 16),
                           __float_as_uint(kn[2]) | (__float_as_uint(kn[3]) << 16),
                           __float_as_uint(kn[4]) | (__float_as_uint(kn[5]) << 16),
                           __float_as_uint(kn[6]) | (__float_as_uint(kn[7]) << 16));
      }
    }
    if (kq == (ns >> 2)) {
      const int e = ns & 3;
      const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      const int sh = (e & 1) ? 16 : 0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t vbits = __float_as_uint(kvnew[D + nb * 16 + r16]) << sh;
        const uint32_t x = vv[nb].x, y = vv[nb].y;
        vv[nb] = e < 2 ? make_uint2((x & keep) | vbits, y) : make_uint2(x, (y & keep) | vbits);
      }
    }
  };
  // Slots at or past the live context may hold stale bits (even NaN) from an
  // earlier owner of the page: their probability is 0, but 0 * NaN is not, so
  // this lane's four V slots 4kq .. 4kq+3 of page pg are zeroed where invalid.
  auto vmask = [&](int pg, uint32_t& mlo, uint32_t& mhi) {
    const int valid = n_tok - pg * 16;
    mlo = 0xFFFFFFFFu;
    mhi = 0xFFFFFFFFu;
    if (valid < 16) {
      const int s0 = 4 * kq;
      mlo = (s0 < valid ? 0x0000FFFFu : 0u) | (s0 + 1 < valid ? 0xFFFF0000u : 0u);
      mhi = (s0 + 2 < valid ? 0x0000FFFFu : 0u) | (s0 + 3 < valid ? 0xFFFF0000u : 0u);
    }
  };
  // Two pages per online-softmax update: their MFMA chains, shuffles and
  // exponentials are independent and overlap. A page index at or past the
  // live context contributes nothing. With two = false (a wave's odd last
  // page) page B is left out altogether: a wave issues one instruction at a
  // time and shares its SIMD's vector unit, so work on an empty page would
  // hold up the waves with two.
  auto compute2 = [&](uint4 (&kA)[NK4], uint2 (&vA)[NB], int pgA, uint4 (&kB)[NK4], uint2 (&vB)[NB],
                      int pgB, bool two) {
    patch(kA, vA, pgA);
    if (two) patch(kB, vB, pgB);
    v4f SA = {0.f, 0.f, 0.f, 0.f}, SB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bf16x8 qs = __builtin_bit_cast(bf16x8, qop[st]);
      SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kA[st]), qs, SA, 0, 0, 0);
      if (two) SB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kB[st]), qs, SB, 0, 0, 0);
    }
    float sa[4], sb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xa = xor8_sum(SA[j]) * scale;
      sa[j] = (pgA * 16 + 4 * kq + j) < n_tok ? xa : NEG_INF;
      sb[j] = NEG_INF;
      if (two) {
        const float xb = xor8_sum(SB[j]) * scale;
        sb[j] = (pgB * 16 + 4 * kq + j) < n_tok ? xb : NEG_INF;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])),
                     fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])));
    mx = xor32_max(xor16_max(mx));
    const float mn = fmaxf(m_run, mx);
    // with no live score yet (mn = -inf) every weight and alpha are 2^-inf = 0
    // against a zero reference (nothing has been accumulated)
    const float mz = mn == NEG_INF ? 0.f : mn;
    const float alpha = exp2_hw(m_run - mz);
    float qa[4], qb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qa[j] = exp2_hw(sa[j] - mz);
      qb[j] = two ? exp2_hw(sb[j] - mz) : 0.f;
    }
    float ps = ((qa[0] + qa[1]) + (qa[2] + qa[3])) + ((qb[0] + qb[1]) + (qb[2] + qb[3]));
    ps = xor32_sum(xor16_sum(ps));
    l_run = l_run * alpha + ps;
    m_run = mn;
    uint32_t pw[4];  // P operand words: page A's tokens 4 kq .. + 3, then page B's
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t hw, lw;
      split2(qa[2 * j], qa[2 * j + 1], hw, lw);
      pw[j] = lo_part ? lw : hw;
      pw[2 + j] = 0u;
      if (two) {
        split2(qb[2 * j], qb[2 * j + 1], hw, lw);
        pw[2 + j] = lo_part ? lw : hw;
      }
    }
    // the scale of output row 4 kq + j, i.e. of head (4 kq + j) & 7, whose
    // alpha every lane with r16 & 7 == head holds (lane head, for one)
    float aj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo4 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), j));
      const float hi4 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 + j));
      aj[j] = (kq & 1) ? hi4 : lo4;
    }
    uint32_t mla, mha, mlb = 0u, mhb = 0u;
    vmask(pgA, mla, mha);
    if (two) vmask(pgB, mlb, mhb);
    // one MFMA 16x16x32 per 16 dims over both pages: reduction index
    // 8 kq + e is token 4 kq + e of page A for e < 4 and of page B for e >= 4,
    // so each lane's own probabilities and V slots form its operands
    const bf16x8 P2 = __builtin_bit_cast(bf16x8, u4v{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[nb][j] *= aj[j];
      const u4v v2 = {vA[nb].x & mla, vA[nb].y & mha, two ? vB[nb].x & mlb : 0u, two ? vB[nb].y & mhb : 0u};
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(P2, __builtin_bit_cast(bf16x8, v2), acc[nb], 0, 0, 0);
    }
  };
  // pages go two at a time: the pair being computed sits in buffers 0 and 1
  // while the pair after it is in flight in buffers 2 and 3; the two halves
  // of the ring alternate roles, and the pair body is instantiated once per
  // half.
  constexpr int NO_PAGE = 1 << 24;  // a page index past any context: contributes nothing
  for (int i0 = 0; i0 < cnt; i0 += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; j += 2) {
      const int i = i0 + j;
      if (i < cnt) {
        if (i + 1 < cnt)
          compute2(kb[j], vb[j], first + i * NWAVE, kb[j + 1], vb[j + 1], first + (i + 1) * NWAVE, true);
        else
          compute2(kb[j], vb[j], first + i * NWAVE, kb[j + 1], vb[j + 1], NO_PAGE, false);
        if (i + NBUF < cnt) load(kb[j], vb[j], first + (i + NBUF) * NWAVE, pid[w + (i + NBUF) * NWAVE]);
        if (i + 1 + NBUF < cnt)
          load(kb[j + 1], vb[j + 1], first + (i + 1 + NBUF) * NWAVE, pid[w + (i + 1 + NBUF) * NWAVE]);
      }
    }
  }
  mark(c, 2);
  if (bad && lane == 0) raise_status(a, DS_BOUNDS, c.ti, (uint32_t)b, 0xFFFFFFFFu);
  // merge the hi/lo rows (row r and r + 8 of the product, lanes L and L ^ 32)
  // and publish this wave's partial in LDS, head fastest: lane (r16, kq < 2)
  // holds heads 4 kq .. + 3 of dim 16 nb + r16, one 16-byte store per nb
  float* Ow = s.att;                      // [NWAVE][D][8]
  float* mw = s.red;                      // [NWAVE][8]
  float* lw = s.out;                      // [NWAVE][8]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float4 o4;
    o4.x = xor32_sum(acc[nb][0]);
    o4.y = xor32_sum(acc[nb][1]);
    o4.z = xor32_sum(acc[nb][2]);
    o4.w = xor32_sum(acc[nb][3]);
    if (kq < 2) *(float4*)(Ow + ((w * D) + nb * 16 + r16) * 8 + 4 * kq) = o4;
  }
  if (lane < 8) {
    mw[w * 8 + lane] = m_run;
    lw[w * 8 + lane] = l_run;
  }
  lds_barrier();
  mark(c, 3);
  // merge over the waves. Every wave forms the 64 scales 2^(m_q,h - M_h) of
  // (wave q, head h) in its lanes (lane 8 q + h; M_h = max_q m_q,h, over lanes
  // of equal h: xor 8, 16, 32) and the heads' sums L_h; thread (dim, head
  // pair) then sums its two heads' outputs with the scales as scalars.
  const int wq = lane >> 3, hw = lane & 7;
  const float mq = hw < HG ? mw[wq * 8 + hw] : NEG_INF;
  float Mh = fmaxf(mq, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(mq), 0x128, 0xF, 0xF, false)));
  Mh = xor32_max(xor16_max(Mh));
  const float e = exp2_hw(mq - (Mh == NEG_INF ? 0.f : Mh));
  const float Lh = xor32_sum(xor16_sum(xor8_sum(e * (hw < HG ? lw[wq * 8 + hw] : 0.f))));
  const int PS = D + 2;
  uint64_t* dst0 = a.part + (size_t)l * a.s_part +
                   (((size_t)b * a.Hkv + g) * a.S_max + split) * HG * PS;
  for (int idx = tid(); idx < (HG + 1) / 2 * D; idx += NT) {
    const int hp = __builtin_amdgcn_readfirstlane(idx / D);  // head pair, uniform in a wave (D % 64 == 0)
    const int dim = idx - hp * D;
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) {
      const float e0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), q * 8 + 2 * hp));
      const float e1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), q * 8 + 2 * hp + 1));
      const float2 v = *(const float2*)(Ow + ((q * D) + dim) * 8 + 2 * hp);
      o0 = fmaf(e0, v.x, o0);
      o1 = fmaf(e1, v.y, o1);
    }
    uint64_t* dst = dst0 + (size_t)(2 * hp) * PS;
    st_tagged(dst + dim, o0, a.epoch);
    if (2 * hp + 1 < HG) st_tagged(dst + PS + dim, o1, a.epoch);
  }
  if (tid() < HG) {  // lanes 0 .. HG-1 of wave 0: head h's M and L
    uint64_t* dst = dst0 + (size_t)tid() * PS;
    st_tagged(dst + D, Mh, a.epoch);
    st_tagged(dst + D + 1, Lh, a.epoch);
  }
  return true;
}

// Batch combine of nh = nd / D whole query heads h .. h + nh - 1 of one kv
// group (d0 = 0, nd = nh D <= NT): per split, the heads' words are one
// contiguous run of nh (D + 2), gathered in pairs into the shared area (no
// pages are staged in a batch plan); thread (head, dim) then merges its
// output over the splits in split order.
static_assert(COMB_BATCH_WORDS == NWAVE * STAGE_CHUNKS * 64 * 4, "batch combine words fill the shared area");
__device__ __forceinline__ bool task_comb_heads(Ctx& c, const Task& t) {
  KAC& a = c.a;
  Smem& s = c.s;
  const int l = t.layer, b = t.a0, h = t.a1, nd = t.a3, S = t.aux, D = a.D;
  const int HG = a.HG, g = h / HG, PS = D + 2, W = nd / D * PS;
  const uint64_t* base = a.part + (size_t)l * a.s_part + ((size_t)b * a.Hkv + g) * a.S_max * HG * PS +
                         (size_t)(h % HG) * PS;
  const size_t sstride = (size_t)HG * PS;
  float* sw = s.att;  // [S][W]
  // W is even and so is every run's workspace word offset
  if (!gather_fn_pairs<8>(c, S * W, [&](int i) {
        const int q = i / W;
        return base + q * sstride + (i - q * W);
      }, sw, 1))
    return false;
  const int tt = tid();
  if (tt < nd) {
    const int hh = tt / D, dim = tt - hh * D;
    const float* col = sw + hh * PS;
    float M = NEG_INF;
    for (int q = 0; q < S; ++q) M = fmaxf(M, col[q * W + D]);
    const float Mz = M == NEG_INF ? 0.f : M;  // split maxima are in log2 units
    float L = 0.f, acc = 0.f;
    for (int q = 0; q < S; ++q) {
      const float mq = col[q * W + D];
      const float e = exp2_hw(mq - Mz);
      L += e * col[q * W + D + 1];
      acc += e * col[q * W + dim];
    }
    const float o = L > 0.f ? acc / L : 0.f;
    st_tagged(a.o + (size_t)l * a.s_o + ((size_t)b * a.Hq + h + hh) * D + dim, o, a.epoch);
  }
  return true;
}

template <bool BATCH>
__device__ __forceinline__ bool task_comb(Ctx& c, const Task& t) {
  if constexpr (BATCH) {
    if (t.a3 > c.a.D) return task_comb_heads(c, t);
  }
  KAC& a = c.a;
  Smem& s = c.s;
  const int l = t.layer, b = t.a0, h = t.a1, d0 = t.a2, nd = t.a3, S = t.aux, D = a.D;
  const int HG = a.HG, g = h / HG, hh = h % HG, PS = D + 2;
  const uint64_t* base = a.part + (size_t)l * a.s_part + ((size_t)b * a.Hkv + g) * a.S_max * HG * PS +
                         (size_t)hh * PS;
  const size_t sstride = (size_t)HG * PS;
  // every split's dims d0 .. d0+nd, max and sum in one batch, in pairs (nd
  // even, every word offset even): split q's words are nd / 2 pairs of dims,
  // then the pair (max, sum), at att[q * (nd + 2) ..]
  const int W = nd + 2;
  float* sw = s.att;
  if (a.trace && tid() == 0) s.tw[2] = now();
  bool ok = true;
  const int WP = W / 2, np = S * WP;
  const uint32_t ob = ws_off(a, base);
  for (int bs = 0; bs < np && ok; bs += 2 * NT) {
    const int t = tid();
    float v[4];
    ok = read_pairs<2>(a, [&](int k) -> uint32_t {
      const int pi = bs + t + k * NT;
      if (pi >= np) return NO_PAIR;
      const int q = pi / WP, j = 2 * (pi - q * WP);
      return ob + 8u * (uint32_t)(q * sstride + (j < nd ? d0 + j : D + (j - nd)));
    }, v, c.t0, c.ti);
    if (ok) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pi = bs + t + k * NT;
        if (pi < np) *(float2*)(sw + 2 * pi) = make_float2(v[2 * k], v[2 * k + 1]);
      }
    }
  }
  if (!ok) s.fail = 1;
  lds_barrier();
  if (a.trace && tid() == 0) s.tw[3] = now();
  if (s.fail) return false;
  // every wave forms the global max M = max_q m_q and the denominator
  // L = sum_q 2^(m_q - M) l_q on its own (split q in lane q, q + 64, ...;
  // the split maxima are in log2 units), so the merge needs no barrier
  // before the weighted sums; thread (sg, dim) then sums 2^(m_q - M) o_q[dim]
  // over its splits q = sg, sg + NG, ...
  const int lane = tid() & 63;
  float M = NEG_INF;
  for (int q = lane; q < S; q += 64) M = fmaxf(M, sw[q * W + nd]);
  M = wave_max_dpp(M);
  const float Mz = M == NEG_INF ? 0.f : M;
  float L = 0.f;
  for (int q = lane; q < S; q += 64) {
    const float mq = sw[q * W + nd];
    L += exp2_hw(mq - Mz) * sw[q * W + nd + 1];
  }
  L = wave_sum(L);
  mark(c, 0);
  const int NG = NT / nd, sg = tid() / nd, dim = tid() % nd;
  float acc = 0.f;
  if (sg < NG)
    for (int q = sg; q < S; q += NG) {
      const float mq = sw[q * W + nd];
      acc += exp2_hw(mq - Mz) * sw[q * W + dim];
    }
  float* red = s.out + 1024;
  int nred = NG;
  if (nd <= 32) {
    // a wave holds 64 / nd split groups of the same nd dims (lanes nd apart):
    // sum them across the wave, leaving one partial per wave
    if (nd <= 8) acc = xor8_sum(acc);
    if (nd <= 16) acc = xor16_sum(acc);
    acc = xor32_sum(acc);
    if ((tid() & 63) < nd) red[(tid() >> 6) * nd + dim] = acc;
    nred = NWAVE;
  } else if (sg < NG) {
    red[sg * nd + dim] = acc;
  }
  mark(c, 1);
  lds_barrier();
  mark(c, 2);
  if (tid() < nd) {
    // nred <= NWAVE partials, read together and summed in order
    float pv[NWAVE];
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) pv[q] = q < nred ? red[q * nd + tid()] : 0.f;
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < NWAVE; ++q)
      if (q < nred) o += pv[q];
    o = L > 0.f ? o / L : 0.f;
    st_tagged(a.o + (size_t)l * a.s_o + ((size_t)b * a.Hq + h) * D + d0 + tid(), o, a.epoch);
  }
  return true;
}

template <int CPL, int TC>
__device__ __forceinline__ bool task_o(Ctx& c, const Task& t) {
  constexpr int RPW = GEMV_REG_CHUNKS / CPL < GEMV_RPW_MAX ? GEMV_REG_CHUNKS / CPL : GEMV_RPW_MAX;
  KAC& a = c.a;
  const int l = t.layer, r0 = t.a1, n = t.a2;
  const int H = a.H, K = a.Hq * a.D;
  const uint16_t* W = a.wo + (size_t)l * H * K;
  Tile<CPL, RPW, TC> tile;
  tile.issue(n, [&](int j) { return (const uint4*)(W + (size_t)(r0 + j) * K); });
  // residual rows (layer input, complete once o is): loaded ahead of the wait
  const int th = tid();
  uint64_t rw = 0;
  if (th < n) {
    if (l == 0) rw = tag_word(bf2f(a.embed[(size_t)token_row(a, 0) * a.H + r0 + th]), a.epoch);
    else rw = ld_tagged(a.x + (size_t)(l - 1) * a.s_x + r0 + th);
  }
  if (!gather_split<8>(c, a.o + (size_t)l * a.s_o, K, c.s.vec, 1)) return false;
  tile.dots(c.s.vec, c.s.out);
  mark(c, 0);
  lds_barrier();
  mark(c, 1);
  bool fail = false;
  if (th < n) {
    const float x = tag_is(rw, a.epoch) ? tag_value(rw) : resid(c, l, 0, r0 + th, &fail);
    st_tagged(a.xa + (size_t)l * a.s_x + r0 + th, x + c.s.out[th], a.epoch);
  }
  for (int j = th + NT; j < n; j += NT) {
    const float x = resid(c, l, 0, r0 + j, &fail);
    st_tagged(a.xa + (size_t)l * a.s_x + r0 + j, x + c.s.out[j], a.epoch);
  }
  return !fail;
}

template <int CPL, int TC>
__device__ __forceinline__ bool task_router(Ctx& c, const Task& t) {
  constexpr int RPW = GEMV_REG_CHUNKS / CPL < GEMV_RPW_MAX ? GEMV_REG_CHUNKS / CPL : GEMV_RPW_MAX;
  KAC& a = c.a;
  const int l = t.layer, b = t.a0, r0 = t.a1, n = t.a2, H = a.H;
  const uint16_t* W = a.router + (size_t)l * a.E * H;
  Tile<CPL, RPW, TC> tile;
  tile.issue(n, [&](int j) { return (const uint4*)(W + (size_t)(r0 + j) * H); });
  Gains gn;
  gn.load(a.ffn_norm + (size_t)l * H, H);
  if (!gather<4>(c, a.xa + (size_t)l * a.s_x + (size_t)b * H, H, c.s.vec, 1, H)) return false;
  norm_pack(c, c.s.vec, H, gn);
  tile.dots(c.s.vec, c.s.out);
  lds_barrier();
  for (int j = tid(); j < n; j += NT)
    st_tagged(a.rlog + (size_t)l * a.s_rlog + (size_t)b * a.E + r0 + j, c.s.out[j], a.epoch);
  return true;
}

// Router logits before the RMSNorm's 1/rms scale (TF_FOLD, batch 1): rows
// r0 .. r0 + n of F [x | o], where x is the layer input, o the attention
// output and F = [W_r diag(g) | W_r diag(g) W_o] (fp32, mk_router_fold). The
// router reads RMSNorm(x + W_o o), so this equals its logits times
// rms(x + W_o o); it needs only what the O tasks need and runs beside them,
// and the expert tasks apply the scale, which they compute for their own
// input anyway. One fp32 GEMV: the rows' chunks are requested up front, the
// inputs gathered behind them, then dots, wave sums and one barrier.
__device__ __forceinline__ bool task_router_fold(Ctx& c, const Task& t) {
  constexpr int FR = 4;  // folded rows per task (the planner gives at most four)
  constexpr int FQ = 4;  // 16-byte chunks of a folded row per thread (H + Hq d <= 8192)
  KAC& a = c.a;
  Smem& s = c.s;
  const int l = t.layer, r0 = t.a1, n = t.a2, H = a.H, K = a.Hq * a.D, KW = (H + K) / 4;
  const float4* F = (const float4*)(a.rfold + ((size_t)l * a.E + r0) * (H + K));
  float4 fr[FR][FQ];
#pragma unroll
  for (int r = 0; r < FR; ++r)
#pragma unroll
    for (int q = 0; q < FQ; ++q) {
      const int i = tid() + q * NT;
      fr[r][q] = r < n && i < KW ? F[(size_t)r * KW + i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  // s.vec = [x (H) | o (K)], fp32
  if (l == 0) {
    const uint16_t* e = a.embed + (size_t)token_row(a, 0) * H;
    for (int i = tid(); i < H; i += NT) s.vec[i] = bf2f(e[i]);
    if (!gather<8>(c, a.o + (size_t)l * a.s_o, K, s.vec + H, 1)) return false;
  } else {
    if (!gather2<6>(c, a.x + (size_t)(l - 1) * a.s_x, H, a.o + (size_t)l * a.s_o, H + K, s.vec, 1)) return false;
  }
  float acc[FR];
#pragma unroll
  for (int r = 0; r < FR; ++r) acc[r] = 0.f;
#pragma unroll
  for (int q = 0; q < FQ; ++q) {
    const int i = tid() + q * NT;
    if (i < KW) {
      const float4 v = *(const float4*)(s.vec + 4 * i);
#pragma unroll
      for (int r = 0; r < FR; ++r) {
        acc[r] = fmaf(fr[r][q].x, v.x, acc[r]);
        acc[r] = fmaf(fr[r][q].y, v.y, acc[r]);
        acc[r] = fmaf(fr[r][q].z, v.z, acc[r]);
        acc[r] = fmaf(fr[r][q].w, v.w, acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < FR; ++r) acc[r] = wave_sum(acc[r]);
  if ((tid() & 63) == 0)
#pragma unroll
    for (int r = 0; r < FR; ++r) s.red[r * NWAVE + (tid() >> 6)] = acc[r];
  lds_barrier();
  if (tid() < n) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) v += s.red[tid() * NWAVE + w];
    st_tagged(a.rlog + (size_t)l * a.s_rlog + r0 + tid(), v, a.epoch);
  }
  return true;
}

// Expert task: route (every expert task computes the same top-k), stream the
// gate/up rows of its slot's expert into registers, SwiGLU them against the
// normalised hidden state and publish the activations; then request the rows
// of the down projection (into the registers the gate/up rows held), read
// every slot's activations behind them and finish its hidden rows:
// x = x_attn + sum_j w_j * W_down[e_j] a_j (fixed j order). Dense FFN: one
// slot, expert 0, weight 1.
template <int CH, int TCH, int CF, int TCF>
__device__ __forceinline__ bool task_expert(Ctx& c, const Task& t) {
  constexpr int RPW_G = GEMV_REG_CHUNKS / CH < GEMV_RPW_MAX ? GEMV_REG_CHUNKS / CH : GEMV_RPW_MAX;
  constexpr int RPW_D = DOWN_CHUNKS / CF < GEMV_RPW_MAX ? DOWN_CHUNKS / CF : GEMV_RPW_MAX;
  KAC& a = c.a;
  Smem& s = c.s;
  const int l = t.layer, b = t.a0, slot = t.aux, f0 = t.a1, nf = t.a2;
  const int r0 = t.a3 >> 16, nr = t.a3 & 0xFFFF;
  const int H = a.H, F = a.F, KK = a.dense ? 1 : a.K, EE = a.dense ? 1 : a.E;
  Gains gn;
  gn.load(a.ffn_norm + (size_t)l * H, H);
  const uint64_t* xa = a.xa + (size_t)l * a.s_x + (size_t)b * H;
  // The router logits and the hidden state after attention in one batch:
  // s.vec = [x_attn (H) | logits (E)]; the gather also leaves the rank keys of
  // the logits, their per-wave maxima and the per-wave sums of squares of
  // x_attn. Then every thread counts the keys ahead of part of the experts
  // (rank = number of keys ahead), and the selection, the residual copy and the
  // norm share the remaining barriers.
  float* lg_ = s.vec + H;
  if (!a.dense) {
    const int E = a.E, E32 = (E + 31) & ~31;
    uint64_t* keys = (uint64_t*)(s.out + 1024);  // [E32] (padding keys 0 rank below all)
    int* partial = (int*)(s.out + 512);          // [parts][E32] (parts * E32 <= 512)
    if (!gather2<5>(c, xa, H, a.rlog + (size_t)l * a.s_rlog + (size_t)b * E, H + E, s.vec, 0, H, keys))
      return false;
    const int parts = E32 <= 128 ? 4 : 2;
    const int chunk = E32 / parts;  // a multiple of 8
    {
      const int te = tid() % E32, part = tid() / E32;
      if (part < parts) {
        const uint64_t mine = keys[te];
        int cnt = 0;
#pragma unroll 2
        for (int e = part * chunk; e < (part + 1) * chunk; e += 8) {
          uint4 q[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) q[i] = *(const uint4*)(keys + e + 2 * i);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            cnt += ((((uint64_t)q[i].y << 32) | q[i].x) > mine) ? 1 : 0;
            cnt += ((((uint64_t)q[i].w << 32) | q[i].z) > mine) ? 1 : 0;
          }
        }
        partial[part * E32 + te] = cnt;
      }
    }
    for (int q = tid(); q < nr; q += NT) s.res[q] = s.vec[r0 + q];
    lds_barrier();
    if (tid() < E) {
      int rank = 0;
      for (int q = 0; q < parts; ++q) rank += partial[q * E32 + tid()];
      if (rank < a.K) s.route_ids[rank] = tid();
    }
    norm_pack(c, s.vec, H, gn);  // its barrier also publishes the selection
  } else {
    if (tid() == 0) {
      s.route_ids[0] = 0;
      s.route_w[0] = 1.f;
      s.route_wn[0] = 1.f;
    }
    if (!gather<4>(c, xa, H, s.vec, 0, H)) return false;
    for (int q = tid(); q < nr; q += NT) s.res[q] = s.vec[r0 + q];
    norm_pack(c, s.vec, H, gn);
  }
  // The routing weights (lanes 0 .. K-1 of wave 0) are formed once the
  // gate/up rows are requested: only the down combine, after later barriers,
  // reads them. Softmax over the selection (renormalised), or the probability
  // of each selected expert (a sum over every expert); folded router logits
  // still lack the RMSNorm's 1/rms of x_attn, whose per-wave sums of squares
  // the gather left in s.red[0 .. NWAVE), beside the per-wave logit maxima.
  auto route_weights = [&]() {
    if (a.dense || tid() >= a.K) return;
    const int E = a.E;
    float sc = 1.f;
    if (t.flags & TF_FOLD) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) tot += s.red[w];
      sc = 1.0f / sqrtf(tot / (float)H + a.eps);
    }
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, s.red[NWAVE + w]);
    const int id = s.route_ids[tid()];
    const float num = expf((lg_[id] - M) * sc);  // softmax numerator
    s.route_w[tid()] = num;  // read back by this wave below (LDS runs a wave's accesses in order)
    __builtin_amdgcn_wave_barrier();
    float div = 0.f;
    if (a.norm_topk) {
      for (int i = 0; i < a.K; ++i) div += s.route_w[i];
    } else {
      for (int e = 0; e < E; ++e) div += expf((lg_[e] - M) * sc);
    }
    const float wn = num / div;
    s.route_wn[tid()] = wn;  // read after later barriers
    if (t.flags & TF_WRITE_TOPK) {
      if (a.topk_ids) a.topk_ids[(size_t)l * a.K + tid()] = id;
      if (a.topk_w) a.topk_w[(size_t)l * a.K + tid()] = wn;
    }
  };
  mark(c, 0);
  const int e = s.route_ids[slot];
  const uint16_t* Wg = a.gate + ((size_t)l * EE + e) * F * H;
  const uint16_t* Wu = a.up + ((size_t)l * EE + e) * F * H;
  const uint16_t* Wd = a.down + (size_t)l * EE * H * F;
  const int capg = (NT / TCH) * RPW_G / 2;   // FFN rows per register tile
  const int capd = (NT / TCF) * RPW_D / KK;  // hidden rows per staged tile
  // The gate/up rows stream into registers; the down rows are requested once
  // the gate/up rows are consumed (a wave's loads complete in issue order, so
  // down rows issued earlier would hold up the gate/up dots), and they stream
  // while the activations of the other expert tasks arrive.
  Tile<CH, RPW_G, TCH> gu;
  Tile<CF, RPW_D, TCF> dn;
  mark(c, 1);
  if (nf == 0) route_weights();
  for (int fc = 0; fc < nf; fc += capg) {
    const int nfc = min(capg, nf - fc);
    gu.issue(2 * nfc, [&](int j) {
      return (const uint4*)(((j & 1) ? Wu : Wg) + (size_t)(f0 + fc + (j >> 1)) * H);
    });
    if (fc == 0) route_weights();
    gu.dots(s.vec, s.out);
    lds_barrier();
    mark(c, 3);
    uint64_t* act = a.act + (size_t)l * a.s_act + ((size_t)b * KK + slot) * F + f0 + fc;
    for (int q = tid(); q < nfc; q += NT) {
      const float yg = s.out[2 * q], yu = s.out[2 * q + 1];
      st_tagged(act + q, yg / (1.0f + expf(-yg)) * yu, a.epoch);
    }
    lds_barrier();
  }
  mark(c, 4);
  if (nr == 0) return true;
  // down part: job j = (hidden row j / KK, slot j % KK); a lane group's slot
  // is fixed because the number of lane groups is a multiple of KK
  for (int rc = 0; rc < nr; rc += capd) {
    const int nrc = min(capd, nr - rc);
    dn.issue(nrc * KK, [&](int j) {
        return (const uint4*)(Wd + ((size_t)s.route_ids[j % KK] * H + r0 + rc + j / KK) * F);
      });
    if (rc == 0) {
      if (!gather_split<12>(c, a.act + (size_t)l * a.s_act + (size_t)b * KK * F, KK * F, s.vec, 1))
        return false;
    }
    mark(c, 5);
    dn.dots(s.vec + (size_t)(dn.lg % KK) * F, s.out);
    lds_barrier();
    mark(c, 7);
    for (int q = tid(); q < nrc; q += NT) {
      float y = 0.f;
      if ((KK & 3) == 0) {
        // KK <= 16 slots in float4 reads (independent of one another, so
        // not each waiting for the last), summed in slot order
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
          if (4 * jb < KK) {
            const float4 wv = *(const float4*)(s.route_wn + 4 * jb);
            const float4 ov = *(const float4*)(s.out + q * KK + 4 * jb);
            y += wv.x * ov.x;
            y += wv.y * ov.y;
            y += wv.z * ov.z;
            y += wv.w * ov.w;
          }
      } else {
        for (int j = 0; j < KK; ++j) y += s.route_wn[j] * s.out[q * KK + j];
      }
      st_tagged(a.x + (size_t)l * a.s_x + (size_t)b * H + r0 + rc + q, s.res[rc + q] + y, a.epoch);
    }
    lds_barrier();
  }
  return true;
}

// LM head tile: rows stream through registers in a ring of LM_RING batches
// of LM_BATCH rows per lane group, so that LM_RING - 1 batches are in flight
// while one is reduced (a batch's registers are refilled as soon as it has
// been reduced: no copy between buffers, which would wait for the batch in
// flight before the next request); every lane group walks the same number
// of batches (rows past the tile's end re-read its last row and are
// ignored), so the loop issues its loads unconditionally.
template <int CPL, int TC>
__device__ __forceinline__ bool task_lm(Ctx& c, const Task& t) {
  constexpr int G = NT / TC;
  KAC& a = c.a;
  Smem& s = c.s;
  const int r0 = t.a1, n = t.a2, H = a.H;
  const int lg = tid() / TC, tc = tid() % TC;
  const int per = (n + G - 1) / G;                       // rows per lane group
  int nb = (per + LM_BATCH - 1) / LM_BATCH;
  nb = nb < LM_RING ? LM_RING : nb;                      // >= LM_RING (the ring is filled up front)
  uint4 W[LM_RING][LM_BATCH][CPL];
  auto row_of = [&](int bi, int r) { return min(lg + (bi * LM_BATCH + r) * G, n - 1); };
  auto issue = [&](uint4 (&w)[LM_BATCH][CPL], int bi) {
#pragma unroll
    for (int r = 0; r < LM_BATCH; ++r) {
      const uint4* p = (const uint4*)(a.lm + (size_t)(r0 + row_of(bi, r)) * H);
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) w[r][cc] = ld_nt(p + tc + cc * TC);
    }
  };
#pragma unroll
  for (int k = 0; k < LM_RING; ++k) issue(W[k], k);
  Gains gn;
  gn.load(a.final_norm, H);
  if (!gather<4>(c, a.x + (size_t)(a.L - 1) * a.s_x, H, s.vec, 1, H)) return false;
  norm_pack(c, s.vec, H, gn);
  uint4 uh[CPL], ul[CPL];
#pragma unroll
  for (int cc = 0; cc < CPL; ++cc) {
    uh[cc] = ((const uint4*)(s.vec + (tc + cc * TC) * 8))[0];
    ul[cc] = ((const uint4*)(s.vec + (tc + cc * TC) * 8))[1];
  }
  // batch bi sits in ring slot bi % LM_RING
  for (int b0 = 0; b0 < nb; b0 += LM_RING) {
#pragma unroll
    for (int k = 0; k < LM_RING; ++k) {
      const int bi = b0 + k;
      if (bi < nb) {
#pragma unroll
        for (int r = 0; r < LM_BATCH; ++r) {
          float sum = 0.f;
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) sum = dot8h(W[k][r][cc], uh[cc], ul[cc], sum);
          sum = group_sum_last<TC>(sum);
          if (tc == TC - 1) s.out[row_of(bi, r)] = sum;
        }
        if (bi + LM_RING < nb) issue(W[k], bi + LM_RING);
      }
    }
  }
  lds_barrier();
  float bv = NEG_INF;
  int bi = 0x7fffffff;
  for (int j = tid(); j < n; j += NT) {
    const float y = s.out[j];
    if (a.logits) a.logits[r0 + j] = y;
    if (a.smp_u) st_tagged(a.lw + r0 + j, y, a.epoch);
    argmax_merge(y, r0 + j, bv, bi);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_merge(ov, oi, bv, bi);
  }
  float* rv = s.red;
  int* ri = (int*)(s.red + NWAVE);
  if ((tid() & 63) == 0) { rv[tid() >> 6] = bv; ri[tid() >> 6] = bi; }
  lds_barrier();
  if (tid() == 0) {
    for (int q = 1; q < NWAVE; ++q)
      argmax_merge(rv[q], ri[q], bv, bi);
    st_tagged(a.lmpart + (size_t)t.a3 * 2, bv, a.epoch);
    st_tagged(a.lmpart + (size_t)t.a3 * 2 + 1, __int_as_float(bi), a.epoch);
  }
  return true;
}

// ------------------------------------------------------------------ sampling
//
// Sampling beyond greedy (the Kinetic book's sampler flags, in llama.cpp's
// default order restricted to top-k, top-p, min-p and temperature, with the
// caller's uniform draw u): the top_k largest logits are found exactly, then
// filtered and drawn from in one wave.

// Order-preserving 64-bit key of logit v of token id: a larger logit ranks
// first, equal logits the lower id; key 0 ranks below every logit.
__device__ __forceinline__ uint64_t tok_key(float v, uint32_t id) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

// Sort the n keys at k (LDS; n a power of two >= 2, written before a
// barrier) into descending order: a bitonic network, every thread taking
// part, a barrier after each stage.
__device__ void lds_sort_desc(uint64_t* k, int n) {
  for (int size = 2; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid(); i < n / 2; i += NT) {
        const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = k[lo], y = k[hi];
        if ((x < y) == desc) {
          k[lo] = y;
          k[hi] = x;
        }
      }
      lds_barrier();
    }
}

__device__ __forceinline__ float wave_scan_incl(float x) {
  const int lane = tid() & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Candidates per sequence: top_k outside 1 .. MK_SAMPLE_TOP_K_MAX is served
// as that maximum; 1 is greedy.
__device__ __forceinline__ int sample_k(KAC& a, int b) {
  int k = a.smp_k[b];
  if (k <= 0 || k > MK_SAMPLE_TOP_K_MAX) k = MK_SAMPLE_TOP_K_MAX;
  return k < a.V ? k : a.V;
}
__device__ __forceinline__ bool sampling(KAC& a, int b) {
  return a.smp_u && a.smp_t[b] > 0.f && sample_k(a, b) > 1;
}

// Sequence b's sampled token into *tok (LDS). The n LM-head tiles hold
// `rows` rows each (the last maybe fewer); tile i's largest logit is value
// tv(i) at row ti(i); the logits themselves are the tagged words a.lw + b*V.
// The K largest tile maxima bound the K largest logits from below, so only
// those K tiles are scanned; logits at or above the running threshold are
// collected, and when the buffer fills its K largest are kept and the
// threshold raised to the K-th. Returns false (uniformly) on deadline or
// another workgroup's failure.
template <class TV, class TI>
__device__ bool sample_seq(Ctx& c, int b, int n, int rows, const TV& tv, const TI& ti, int* tok) {
  KAC& a = c.a;
  Smem& s = c.s;
  constexpr int NKEY = 4096, CAP = 8192, PER = 8, ROUND = NT * PER;
  static_assert(sizeof(Smem::stage) >= (NKEY + CAP) * sizeof(uint64_t), "sampling keys exceed the shared area");
  static_assert(CAP - ROUND >= MK_SAMPLE_TOP_K_MAX, "a round must fit after keeping the top k");
  uint64_t* keys = (uint64_t*)s.stage;  // tile maxima (NKEY), then candidates (CAP): 96 KB
  uint64_t* cand = keys + NKEY;
  int* tiles = (int*)s.res;
  int* cnt = (int*)s.out;
  const int K = sample_k(a, b);
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  for (int i = tid(); i < n2; i += NT) keys[i] = i < n ? tok_key(tv(i), (uint32_t)ti(i)) : 0ull;
  lds_barrier();
  lds_sort_desc(keys, n2);
  const int nt = n < K ? n : K;
  uint64_t thr = n <= K ? 0ull : keys[K - 1];
  if (tid() < nt) tiles[tid()] = (int)(key_id(keys[tid()]) / (uint32_t)rows);
  if (tid() == 0) *cnt = 0;
  lds_barrier();
  // the nt tiles' rows as one index space (element e: tile e / rows, row
  // e % rows, past the vocabulary in the last tile: none), PER words per
  // thread per round
  const uint64_t* lw = a.lw + (size_t)b * a.V;
  const int total = nt * rows;
  for (int base = 0; base < total; base += ROUND) {
    float v[PER];
    const bool ok = read_words<PER>(a, [&](int k) -> const uint64_t* {
      const int e = base + tid() + k * NT;
      if (e >= total) return nullptr;
      const int r = tiles[e / rows] * rows + e % rows;
      return r < a.V ? lw + r : nullptr;
    }, v, c.t0, c.ti);
    if (!ok) s.fail = 1;
    if (ok)
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int e = base + tid() + k * NT;
        const int r = e < total ? tiles[e / rows] * rows + e % rows : a.V;
        if (r < a.V) {
          const uint64_t key = tok_key(v[k], (uint32_t)r);
          if (key >= thr) cand[atomicAdd(cnt, 1)] = key;
        }
      }
    lds_barrier();
    if (s.fail) return false;
    const int m = *cnt;
    if (m > CAP - ROUND) {  // keep the K largest, raise the threshold
      int m2 = 2;
      while (m2 < m) m2 <<= 1;
      for (int i = m + tid(); i < m2; i += NT) cand[i] = 0ull;
      lds_barrier();
      lds_sort_desc(cand, m2);
      thr = cand[K - 1];
      if (tid() == 0) *cnt = K;
      lds_barrier();
    }
  }
  {
    const int m = *cnt;  // >= K: the K tile maxima themselves were collected
    int m2 = 2;
    while (m2 < m) m2 <<= 1;
    for (int i = m + tid(); i < m2; i += NT) cand[i] = 0ull;
    lds_barrier();
    lds_sort_desc(cand, m2);
  }
  if (tid() < 64) {
    const int lane = tid();
    const bool in = lane < K;
    const uint64_t key = in ? cand[lane] : 0ull;
    const float z = in ? key_value(key) : 0.f;
    const float z0 = key_value(cand[0]);
    const float T = a.smp_t[b], P = a.smp_p[b], MP = a.smp_minp[b], u = a.smp_u[b];
    // top-p: softmax over the candidates at temperature 1, most likely first
    const float e = in ? expf(z - z0) : 0.f;
    const float p = e / wave_sum(e);
    const float before = wave_scan_incl(p) - p;
    bool keep = in && (lane == 0 || P >= 1.f || before < P);
    // min-p: at least min_p times as likely as the best (the best always stays)
    if (MP > 0.f) keep = keep && (lane == 0 || z >= z0 + logf(MP));
    // temperature, then the draw
    const float w = keep ? expf((z - z0) / T) : 0.f;
    const float cw = wave_scan_incl(w);
    const float W = __shfl(cw, 63, 64);
    const uint64_t hit = __ballot(keep && cw > u * W);
    const uint64_t kept = __ballot(keep);
    const int pick = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(kept);
    if (lane == pick) *tok = (int)key_id(key);
  }
  lds_barrier();
  return true;
}

__device__ __forceinline__ bool task_final(Ctx& c, const Task& t) {
  KAC& a = c.a;
  Smem& s = c.s;
  const int n = t.a0;
  if (!gather<2>(c, a.lmpart, 2 * n, s.vec, 1)) return false;
  float bv = NEG_INF;
  int bi = 0x7fffffff;
  for (int q = tid(); q < n; q += NT) {
    const float v = s.vec[2 * q];
    const int i = __float_as_int(s.vec[2 * q + 1]);
    argmax_merge(v, i, bv, bi);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_merge(ov, oi, bv, bi);
  }
  float* rv = s.red;
  int* ri = (int*)(s.red + NWAVE);
  if ((tid() & 63) == 0) { rv[tid() >> 6] = bv; ri[tid() >> 6] = bi; }
  lds_barrier();
  if (sampling(a, 0)) {
    int* tok = &s.tok;
    if (!sample_seq(c, 0, n, t.a2, [&](int i) { return s.vec[2 * i]; },
                    [&](int i) { return __float_as_int(s.vec[2 * i + 1]); }, tok))
      return false;
    if (tid() == 0) {
      a.tok_out[0] = *tok;
      a.seq_lens[0] = a.seq_lens[0] + 1;
    }
    return true;
  }
  if (tid() == 0) {
    for (int q = 1; q < NWAVE; ++q)
      argmax_merge(rv[q], ri[q], bv, bi);
    a.tok_out[0] = bi;
    a.seq_lens[0] = a.seq_lens[0] + 1;
  }
  return true;
}

// ------------------------------------------------------------------ batch tasks
//
// A batch of B = 2 .. 32 sequences (continuous batching over one shared page
// pool) runs the dense projections (QKV, O, LM head) as MFMA tiles: 16 weight
// rows x 16 or 32 sequences per v_mfma_f32_16x16x32_bf16, the weights as the
// A operand straight from HBM and the sequences' inputs as the B operand from
// LDS. Inputs are fp32; they enter the MFMA as bf16 hi + lo parts (two MFMAs
// per product, each bf16 x bf16 product exact in fp32), which keeps every
// projection at fp32-level accuracy. RMSNorm is applied as x * g on the way
// into LDS and the per-sequence scale 1/sqrt(mean(x^2) + eps) on the way out
// (W (s x * g) = s W (x * g)). Attention and the split combine are the batch-1
// bodies, per sequence. The router and top-k run per sequence; expert tasks
// take the sequences routed to their expert (any number, in groups) so that
// each selected expert's weights stream once per step.


// LDS of an MFMA batch tile, overlaid on the vector and staging areas.
// Activation panel chunk (st, cb, lane) holds 8 k values 32 st + 8 (lane / 16)
// .. + 7 of sequence 16 cb + lane % 16: one ds_read_b128 per lane gives the B
// operand of k-step st for column block cb.
struct MtLds {
  uint4 hi[2][8 * 2 * 64];             // two panels of bf16 hi parts
  uint4 lo[2][8 * 2 * 64];             // and of lo parts
  float red[NWAVE][2][4][64];          // k-split partial accumulators
  float ss[NT];                        // sum-of-squares partials
  float scale[MAX_BATCH];              // per-sequence norm scale
  float ssum[MAX_BATCH];               // per-sequence sum of squares of the tile's inputs
  float out[MT_MAX_BLOCKS * 16][MAX_BATCH];  // finished tile: [row][sequence]
};
static_assert(sizeof(MtLds) <= sizeof(float) * LDS_VEC + sizeof(uint4) * NWAVE * STAGE_CHUNKS * 64,
              "MFMA tile LDS exceeds the overlaid areas");

// Input of an MFMA tile: sequence b's K values at words + b * ld (tagged fp32)
// or, when words is null, the embedding row of sequence b's token (bf16).
// gain: bf16 norm gains applied on the way in (null: none); norm: scale each
// sequence's results by 1/sqrt(mean(x^2) + eps).
struct MtSrc {
  const uint64_t* words;
  int64_t ld;
  const uint16_t* gain;
  bool norm;
  int k0 = 0;  // embedding rows: first column read (rows of ld elements)
};

// out[r][b] = sum_k W[row r][k] * x_b[k] (normalised per MtSrc) for r < R <=
// 16 MT_MAX_BLOCKS, b < B, into MtLds::out. rowptr(r) gives weight row r
// (bf16, K elements, K a multiple of MT_KP). Waves split the row blocks and,
// where there are fewer than 8 blocks, the k-steps of every panel (ks waves
// per block, summed in fixed order). Weights of two panels ahead and the
// next panel's inputs are in flight while a panel is multiplied. Every load
// is issued unconditionally (unused slots re-read a valid address) so that
// the wait counts do not depend on the branch taken.
template <class RowPtr>
__device__ __forceinline__ bool mt_tile(Ctx& c, int R, int K, const RowPtr& rowptr, const MtSrc& src) {
  KAC& a = c.a;
  MtLds& P = *(MtLds*)&c.s;
  const int t = tid(), lane = t & 63, w = t >> 6;
  const int B = a.B, ncb = B > 16 ? 2 : 1, npan = K / MT_KP;
  const int nrb = (R + 15) >> 4;
  const int nrbp = nrb <= 1 ? 1 : nrb <= 2 ? 2 : nrb <= 4 ? 4 : 8;
  const int ks = NWAVE / nrbp, nsl = NWAVE / ks;  // waves per row block, k-steps per panel per wave
  const int rb = w / ks, kp = w % ks;
  const bool active = rb < nrb;
  const uint16_t* wrow = rowptr(min(rb * 16 + (lane & 15), R - 1)) + 8 * (lane >> 4);
  auto issue_w = [&](int p, uint4 (&wr)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int st = kp + (s < nsl ? s : 0) * ks;
      wr[s] = ld_nt((const uint4*)(wrow + p * MT_KP + st * 32));
    }
  };
  // panel fill: wave w fills column block cb_t = w & 1, k-group kg = w >> 1
  // of every k-step; lanes 4 m .. 4 m + 3 hold words 2 jw, 2 jw + 1 of the
  // chunk (8 k values) of sequence 16 cb_t + m, so each load instruction reads
  // whole 64-byte runs of 16 sequences, two tagged words per lane
  const int cb_t = w & 1, kg = w >> 1, m4 = lane >> 2, jw = lane & 3;
  const int seq = cb_t * 16 + m4;
  const bool sv = seq < B;
  const int sq = sv ? seq : 0;
  const int kl = 8 * kg + 2 * jw;  // this lane's first k within a k-step
  const bool xw = src.words != nullptr;
  const tag_rsrc rx = tagged_rsrc(xw ? src.words : (const uint64_t*)a.embed,
                                  xw ? (uint32_t)(((size_t)(B - 1) * src.ld + K) * 8) : 0u);
  const uint32_t xoff = (uint32_t)(((size_t)sq * src.ld + kl) * 8);
  const uint16_t* xe = xw ? nullptr : a.embed + (size_t)token_row(a, sq) * src.ld + src.k0 + kl;
  float ss = 0.f;
  struct ActRegs { uint4 v[8]; uint32_t e[8]; uint32_t g[8]; };
  auto issue_act = [&](int p, ActRegs& r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k0 = p * MT_KP + i * 32;
      if (xw) r.v[i] = ld_tagged2(rx, xoff + (uint32_t)k0 * 8u);
      else r.e[i] = *(const uint32_t*)(xe + k0);
      r.g[i] = src.gain ? *(const uint32_t*)(src.gain + k0 + kl) : 0x3F803F80u;
    }
  };
  // check the words' tags (re-reading stale pairs), then convert into panel bi
  auto finish_act = [&](int p, ActRegs& r, int bi) -> bool {
    if (xw && sv) {
      const uint32_t ep = a.epoch;
      uint32_t stale = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) stale |= tag2_is(r.v[i], ep) ? 0u : (1u << i);
      uint32_t it = 0;
      while (stale) {
        __builtin_amdgcn_s_sleep(2);
        tagged_reload_fence();
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (stale & (1u << i)) r.v[i] = ld_tagged2(rx, xoff + (uint32_t)(p * MT_KP + i * 32) * 8u);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((stale & (1u << i)) && tag2_is(r.v[i], ep)) stale &= ~(1u << i);
        if (stale && (++it & 31u) == 0u) {
          if (aborted(a)) return false;
          if (now() - c.t0 > a.timeout_ticks) {
            raise_status(a, DS_TIMEOUT, c.ti, (uint32_t)seq, 0xFFFFFFFEu);
            return false;
          }
        }
      }
    }
    uint32_t* ph = (uint32_t*)P.hi[bi];
    uint32_t* pl = (uint32_t*)P.lo[bi];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x0, x1;
      if (xw) {
        x0 = sv ? __uint_as_float(r.v[i].x) : 0.f;
        x1 = sv ? __uint_as_float(r.v[i].z) : 0.f;
      } else {
        x0 = sv ? bf_lo(r.e[i]) : 0.f;
        x1 = sv ? bf_hi(r.e[i]) : 0.f;
      }
      ss = fmaf(x0, x0, ss);
      ss = fmaf(x1, x1, ss);
      x0 *= bf_lo(r.g[i]);
      x1 *= bf_hi(r.g[i]);
      uint32_t hw, lw;
      split2(x0, x1, hw, lw);
      const int word = ((i * 2 + cb_t) * 64 + kg * 16 + m4) * 4 + jw;
      ph[word] = hw;
      pl[word] = lw;
    }
    return true;
  };
  v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  auto compute = [&](const uint4 (&wr)[8], int bi) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < nsl) {
        const int st = kp + s * ks;
        const bf16x8 A = __builtin_bit_cast(bf16x8, wr[s]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          if (cb < ncb) {
            const uint4 bh = P.hi[bi][(st * 2 + cb) * 64 + lane], bl = P.lo[bi][(st * 2 + cb) * 64 + lane];
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bh), acc[cb], 0, 0, 0);
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bl), acc[cb], 0, 0, 0);
          }
      }
  };
  // one panel: next inputs in flight, multiply, refill weights two panels
  // ahead, land the next inputs in the other buffer; uniform failure
  auto panel = [&](int p, uint4 (&wr)[8], int bi) -> bool {
    ActRegs r;
    const bool more = p + 1 < npan;
    if (more) issue_act(p + 1, r);
    if (active) compute(wr, bi);
    if (p + 2 < npan) issue_w(p + 2, wr);
    if (more && !finish_act(p + 1, r, bi ^ 1)) c.s.fail = 1;
    lds_barrier();
    return c.s.fail == 0;
  };
  uint4 wA[8], wB[8];
  issue_w(0, wA);
  if (npan > 1) issue_w(1, wB);
  {
    ActRegs r;
    issue_act(0, r);
    if (!finish_act(0, r, 0)) c.s.fail = 1;
    lds_barrier();
    if (c.s.fail) return false;
  }
  for (int p = 0; p < npan; p += 2) {
    if (!panel(p, wA, 0)) return false;
    if (p + 1 < npan && !panel(p + 1, wB, 1)) return false;
  }
  // per-sequence scale: the 16 threads of a sequence, in a fixed order
  P.ss[t] = ss;
  if (active && kp > 0) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) P.red[w][cb][j][lane] = acc[cb][j];
  }
  lds_barrier();
  if (t < MAX_BATCH) {
    float tot = 0.f;
    const int cb = t >> 4, s16 = t & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) tot += P.ss[(2 * q + cb) * 64 + 4 * s16 + j];
    P.scale[t] = src.norm ? 1.0f / sqrtf(tot / (float)K + a.eps) : 1.f;
    P.ssum[t] = tot;
  }
  lds_barrier();
  if (active && kp == 0) {
    for (int q = 1; q < ks; ++q)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[cb][j] += P.red[w + q][cb][j][lane];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = rb * 16 + 4 * (lane >> 4) + j, sb = cb * 16 + (lane & 15);
        P.out[row][sb] = acc[cb][j] * P.scale[sb];
      }
  }
  lds_barrier();
  return true;
}

// Context bound of sequence b (from the plan image).
__device__ __forceinline__ int seq_bound(KAC& a, int b) { return a.seq_bound ? a.seq_bound[b] : a.bound; }

// QKV rows of one kv group for every sequence, then the rotary epilogue, the
// new K/V in the step's words and the KV append at each sequence's position.
__device__ __forceinline__ bool task_bqkv(Ctx& c, const Task& t) {
  KAC& a = c.a;
  const int l = t.layer, g = t.a0, p0 = t.a1, np = t.a2, H = a.H, D = a.D;
  const int QR = (a.Hq + 2 * a.Hkv) * D;
  const uint16_t* W = a.wqkv + (size_t)l * QR * H;
  // reduction block kb of KB over the hidden state (KB = 1: the whole row)
  const int kb = t.a3 & 0xFF, KB = max(1, t.a3 >> 8), Kb = H / KB, k0 = kb * Kb;
  MtSrc src{l == 0 ? nullptr : a.x + (size_t)(l - 1) * a.s_x + k0, H, a.attn_norm + (size_t)l * H + k0,
            KB == 1, k0};
  if (a.trace && tid() == 0) c.s.tw[2] = now();
  if (!mt_tile(c, 2 * np, Kb, [&](int j) {
        int head, i, row;
        qkv_pair(p0 + (j >> 1), g, a.HG, D, a.Hq, a.Hkv, &head, &i, &row);
        return W + (size_t)(row + (j & 1) * (D / 2)) * H + k0;
      }, src))
    return false;
  if (a.trace && tid() == 0) c.s.tw[3] = now();
  MtLds& P = *(MtLds*)&c.s;
  if (KB > 1) {
    // partial record of (block kb, row block rb, sequence b): the rows, the
    // sum of squares of this block's inputs, a pad word
    const int nrb_g = ((a.HG * D + 2 * D) / 2 + BQKV_PAIRS - 1) / BQKV_PAIRS;
    const int nrb = a.Hkv * nrb_g, rb = g * nrb_g + p0 / BQKV_PAIRS;
    const int W2 = 2 * np + 2;
    uint64_t* qp = a.qpart + (size_t)l * a.s_qpart;
    auto rec = [&](int q, int b) { return qp + (((size_t)q * nrb + rb) * a.B + b) * QPART_STRIDE; };
    if (kb > 0) {
      for (int idx = tid(); idx < a.B * W2; idx += NT) {
        const int b = idx / W2, r = idx - b * W2;
        const float v = r < 2 * np ? P.out[r][b] : (r == 2 * np ? P.ssum[b] : 0.f);
        st_tagged(rec(kb - 1, b) + r, v, a.epoch);
      }
      return true;
    }
    // block 0: add the other blocks' partial rows and sums of squares (in
    // block order), then normalise; the tile's panel area is free by now
    float* red = (float*)P.hi;  // word (q, b, r) at red[(q * B + b) * W2 + r]
    const int bw = a.B * W2;
    if (!gather_fn_pairs<8>(c, (KB - 1) * bw, [&](int i) {
          const int q = i / bw, rem = i - q * bw, b = rem / W2;
          return rec(q, b) + (rem - b * W2);
        }, red, 0))
      return false;
    if (tid() < a.B) {
      float ss = P.ssum[tid()];
      for (int q = 0; q < KB - 1; ++q) ss += red[(q * a.B + tid()) * W2 + 2 * np];
      P.scale[tid()] = 1.0f / sqrtf(ss / (float)H + a.eps);
    }
    lds_barrier();
    for (int idx = tid(); idx < 2 * np * a.B; idx += NT) {
      const int r = idx / a.B, b = idx - r * a.B;
      float y = P.out[r][b];
      for (int q = 0; q < KB - 1; ++q) y += red[(q * a.B + b) * W2 + r];
      P.out[r][b] = y * P.scale[b];
    }
    lds_barrier();
  }
  // With TF_PREFILL the chunk's later rows read these pool slots in this
  // step: every thread writes its slots, releases them, then stores the
  // tagged words those rows wait on (one pass per kind of write).
  const bool pf = (t.flags & TF_PREFILL) != 0;
  for (int pass = pf ? 0 : 1; pass < 2; ++pass) {
    for (int idx = tid(); idx < np * a.B; idx += NT) {
      const int q = idx / a.B, b = idx - q * a.B;
      const int pos = a.seq_lens[b];
      const bool in_bounds = pos >= 0 && pos + 1 <= seq_bound(a, b) && pos < a.n_rope;
      const int pc = in_bounds ? pos : 0;
      const int32_t phys = a.page_table[(size_t)b * a.max_pages + (pc >> 4)];
      int head, i, row;
      const int sec = qkv_pair(p0 + q, g, a.HG, D, a.Hq, a.Hkv, &head, &i, &row);
      const float y0 = P.out[2 * q][b], y1 = P.out[2 * q + 1][b];
      float r0 = y0, r1 = y1;
      if (sec < 2) {
        const float cs = a.rope_cos[(size_t)pc * (D / 2) + i], sn = a.rope_sin[(size_t)pc * (D / 2) + i];
        r0 = y0 * cs - y1 * sn;
        r1 = y1 * cs + y0 * sn;
      }
      if (sec == 0) {
        if (pass == 1) {
          uint64_t* qd = a.q + (size_t)l * a.s_q + ((size_t)b * a.Hq + head) * D;
          st_tagged(qd + i, r0, a.epoch);
          st_tagged(qd + i + D / 2, r1, a.epoch);
        }
      } else {
        const uint32_t bb = pk_bf16(r0, r1), b0 = bb & 0xFFFFu, b1 = bb >> 16;
        if (pass == 1) {
          uint64_t* kn = a.kvn + (size_t)l * a.s_kvn + (((size_t)b * a.Hkv + g) * 2 + (sec - 1)) * D;
          st_tagged(kn + i, __uint_as_float(b0), a.epoch);
          st_tagged(kn + i + D / 2, __uint_as_float(b1), a.epoch);
        }
        if (pass == 0 || !pf) {
          const bool page_ok = in_bounds && phys >= 0 && phys < a.n_pages;
          if (!page_ok) raise_status(a, DS_BOUNDS, c.ti, (uint32_t)pos, (uint32_t)phys);
          else {
            uint16_t* base = a.pool + (size_t)phys * a.page_stride + (size_t)l * a.layer_stride +
                             (size_t)g * 2 * 16 * D;
            const int slot = pos & 15;
            if (sec == 1) {
              base[kv_k_offset(slot, i)] = (uint16_t)b0;
              base[kv_k_offset(slot, i + D / 2)] = (uint16_t)b1;
            } else {
              base[kv_v_offset(slot, i, D)] = (uint16_t)b0;
              base[kv_v_offset(slot, i + D / 2, D)] = (uint16_t)b1;
            }
          }
        }
      }
    }
    if (pass == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  }
  return true;
}

// Batch O projection. A tile: W_o rows a1 .. a1 + a2 of every sequence over
// reduction block kb (a0) of the a3 blocks of the attention output; with one
// block it adds the residual (the layer's input) and finishes the rows, else
// it publishes its partial sums (OPART, slot kb). A summing task (TF_REDUCE)
// finishes rows a1 .. a1 + a2: it gathers the a3 blocks' partial sums of
// those rows and their residual in one batch and adds them in block order,
// so the reduction is spread over as many tasks as the tiles (a single task
// per row block gathering every other block's rows took ~20 us at batch 32).
__device__ __forceinline__ bool task_bo(Ctx& c, const Task& t) {
  KAC& a = c.a;
  const int l = t.layer, kb = t.a0, r0 = t.a1, n = t.a2, KB = t.a3 > 0 ? t.a3 : 1;
  const int H = a.H, K = a.Hq * a.D, B = a.B;
  const uint64_t* xin = l > 0 ? a.x + (size_t)(l - 1) * a.s_x : nullptr;
  const uint64_t* op = a.opart + (size_t)l * a.s_opart;
  if (t.flags & TF_REDUCE) {
    // rows r0 .. r0 + n: the KB blocks' partial sums and the residual; word
    // (q, b, r) at red[(q * B + b) * n + r], q = 0 the residual (layer > 0),
    // q >= 1 the partial of block q - 1; summed in block order
    float* red = c.s.vec;
    const int bn = B * n;
    auto waddr = [&](int i) -> const uint64_t* {
      const int q = i / bn, rem = i - q * bn, b = rem / n, r = rem - b * n;
      if (q == 0) return xin ? xin + (size_t)b * H + r0 + r : nullptr;
      return op + ((size_t)(q - 1) * B + b) * H + r0 + r;
    };
    // pairs of rows (r, r + 1): even n, r0 and H keep every pair in one row range
    const bool pairs = !((n | r0 | H) & 1) && !((ws_off(a, op) >> 3) & 1) && !(xin && ((ws_off(a, xin) >> 3) & 1));
    if (!(pairs ? gather_fn_pairs<16>(c, (KB + 1) * bn, waddr, red, 0)
                : gather_fn<8>(c, (KB + 1) * bn, waddr, red, 0)))
      return false;
    for (int idx = tid(); idx < bn; idx += NT) {
      const int r = idx / B, b = idx - r * B;
      float y = red[(B + b) * n + r];
      for (int q = 2; q <= KB; ++q) y += red[(q * B + b) * n + r];
      const float x = l > 0 ? red[b * n + r] : bf2f(a.embed[(size_t)token_row(a, b) * H + r0 + r]);
      st_tagged(a.xa + (size_t)l * a.s_x + (size_t)b * H + r0 + r, x + y, a.epoch);
    }
    return true;
  }
  const int Kb = K / KB, k0 = kb * Kb;
  const uint16_t* W = a.wo + (size_t)l * H * K + k0;
  MtSrc src{a.o + (size_t)l * a.s_o + k0, K, nullptr, false};
  if (a.trace && tid() == 0) c.s.tw[2] = now();
  if (!mt_tile(c, n, Kb, [&](int j) { return W + (size_t)(r0 + j) * K; }, src)) return false;
  if (a.trace && tid() == 0) c.s.tw[3] = now();
  MtLds& P = *(MtLds*)&c.s;
  if (KB > 1) {  // publish the tile's partial sums (block kb)
    uint64_t* dst = a.opart + (size_t)l * a.s_opart + (size_t)kb * B * H;
    for (int idx = tid(); idx < n * B; idx += NT) {
      const int r = idx / B, b = idx - r * B;
      st_tagged(dst + (size_t)b * H + r0 + r, P.out[r][b], a.epoch);
    }
    return true;
  }
  // one block: the tile finishes its rows with the residual
  float* res = (float*)P.hi;  // the tile's panel area is free by now
  if (!gather_fn<8>(c, B * n, [&](int i) -> const uint64_t* {
        const int b = i / n, r = i - b * n;
        return xin ? xin + (size_t)b * H + r0 + r : nullptr;
      }, res, 0))
    return false;
  for (int idx = tid(); idx < n * B; idx += NT) {
    const int r = idx / B, b = idx - r * B;
    const float x = l > 0 ? res[b * n + r] : bf2f(a.embed[(size_t)token_row(a, b) * H + r0 + r]);
    st_tagged(a.xa + (size_t)l * a.s_x + (size_t)b * H + r0 + r, x + P.out[r][b], a.epoch);
  }
  return true;
}

// Router rows, softmax and top-k of sequence b: router logits, and per slot
// the selected expert and its (renormalised) weight as route words.
template <int CPL, int TC>
__device__ __forceinline__ bool task_topk(Ctx& c, const Task& t) {
  constexpr int RPW = GEMV_REG_CHUNKS / CPL < GEMV_RPW_MAX ? GEMV_REG_CHUNKS / CPL : GEMV_RPW_MAX;
  constexpr int CAP = (NT / TC) * RPW;
  KAC& a = c.a;
  Smem& s = c.s;
  const int l = t.layer, b = t.a0, H = a.H, E = a.E;
  const bool read = (t.flags & TF_LOGITS) != 0;  // the router tasks computed the logits
  if (read) {
    if (!gather<4>(c, a.rlog + (size_t)l * a.s_rlog + (size_t)b * E, E, s.out, 1)) return false;
  } else {
    const uint16_t* W = a.router + (size_t)l * E * H;
    Tile<CPL, RPW, TC> tile;
    tile.issue(min(CAP, E), [&](int j) { return (const uint4*)(W + (size_t)j * H); });
    Gains gn;
    gn.load(a.ffn_norm + (size_t)l * H, H);
    if (!gather<4>(c, a.xa + (size_t)l * a.s_x + (size_t)b * H, H, s.vec, 1)) return false;
    rmsnorm_pack(c, s.vec, H, gn);
    tile.dots(s.vec, s.out);
    for (int r0 = CAP; r0 < E; r0 += CAP) {
      tile.issue(min(CAP, E - r0), [&](int j) { return (const uint4*)(W + (size_t)(r0 + j) * H); });
      tile.dots(s.vec, s.out + r0);
    }
    lds_barrier();
  }
  route(c, s.out);
  const float div = route_div(a, s);
  if (!read)
    for (int e = tid(); e < E; e += NT)
      st_tagged(a.rlog + (size_t)l * a.s_rlog + (size_t)b * E + e, s.out[e], a.epoch);
  if (tid() < a.K) {
    const int j = tid(), id = s.route_ids[j];
    const float wj = s.route_w[j] / div;
    uint64_t* rw = a.route + (size_t)l * a.s_route + ((size_t)b * a.K + j) * 2;
    st_tagged(rw, __int_as_float(id), a.epoch);
    st_tagged(rw + 1, wj, a.epoch);
    if (a.topk_ids) a.topk_ids[((size_t)l * a.B + b) * a.K + j] = id;
    if (a.topk_w) a.topk_w[((size_t)l * a.B + b) * a.K + j] = wj;
  }
  return true;
}

// Expert GEMM on MFMA: R weight rows (bf16, K elements each) against up to
// 16 input columns held in LDS in split form (column n at in + n * ld
// floats, chunk c = elements 8c .. 8c+7 as 4 words of bf16 hi pairs then 4
// words of lo pairs): out(r, n) = sum_k W[r][k] x_n[k]. Waves take pairs of
// 16-row blocks round-robin; per k-step of 32 each lane loads 16 bytes of
// the A operand (row r16 of the block, k 32 st + 8 kq .. + 7): this lane's
// 16 bytes of k-step 0 of row block rb are at base(rb), those of k-step st
// stride uint4 further on (row-major weights: 16 rows x 64 bytes per wave
// load; the tile order of mk_expert_tile: one contiguous kilobyte). Each
// lane reads that chunk of column r16 (hi and lo: two B operands),
// two MFMA 16x16x32 per block. Weights of the next KC k-steps are in flight
// while a group is multiplied. epi(rb, acc) receives block rb's accumulators:
// lane (n = r16, kq) holds rows 16 rb + 4 kq + j, j < 4, of column n (n >=
// ncols repeats column ncols - 1 and is to be ignored). K % (32 KC) == 0.
template <class RowBase, class Epi>
__device__ __forceinline__ void mfma_rows(int R, int K, const RowBase& base, int stride, const float* in, int ld,
                                          int ncols, const Epi& epi) {
  constexpr int KC = 8;
  const int lane = tid() & 63, w = tid() >> 6, r16 = lane & 15, kq = lane >> 4;
  const int nrb = (R + 15) >> 4, nks = K >> 5;
  const float* inn = in + (size_t)min(r16, ncols - 1) * ld + 8 * kq;
  for (int rbA = 2 * w; rbA < nrb; rbA += 2 * NWAVE) {
    const int rbB = min(rbA + 1, nrb - 1);
    const uint4* wa = base(rbA);
    const uint4* wb = base(rbB);
    v4f accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
    uint4 xa[KC], xb[KC], ya[KC], yb[KC];
    auto load = [&](uint4 (&pa)[KC], uint4 (&pb)[KC], int s0) {
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        pa[i] = ld_nt(wa + stride * (s0 + i));
        pb[i] = ld_nt(wb + stride * (s0 + i));
      }
    };
    auto mul = [&](const uint4 (&pa)[KC], const uint4 (&pb)[KC], int s0) {
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const uint4* ip = (const uint4*)(inn + 32 * (s0 + i));
        const bf16x8 hi = __builtin_bit_cast(bf16x8, ip[0]), lo = __builtin_bit_cast(bf16x8, ip[1]);
        const bf16x8 A = __builtin_bit_cast(bf16x8, pa[i]), Bw = __builtin_bit_cast(bf16x8, pb[i]);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, hi, accA, 0, 0, 0);
        accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, lo, accA, 0, 0, 0);
        accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Bw, hi, accB, 0, 0, 0);
        accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Bw, lo, accB, 0, 0, 0);
      }
    };
    load(xa, xb, 0);
    for (int s0 = 0; s0 < nks; s0 += 2 * KC) {
      if (s0 + KC < nks) load(ya, yb, s0 + KC);
      mul(xa, xb, s0);
      if (s0 + 2 * KC < nks) load(xa, xb, s0 + 2 * KC);
      if (s0 + KC < nks) mul(ya, yb, s0 + KC);
    }
    epi(rbA, accA);
    if (rbB != rbA) epi(rbB, accB);
  }
}

// Column stride (floats) of an expert task's inputs in LDS: a padding of 8
// floats shifts consecutive columns by 8 banks.
__device__ __forceinline__ int exp_ld(int K) { return K + 8; }

// LDS of a batch expert task (overlaid on the vector and staging areas):
// the inputs of one group of routed sequences in split form, and the routed
// (sequence, slot) list.
struct ExpLds {
  float in[EXP_GROUP * (2048 + 8)];
  float ids[MAX_BATCH * 16];
  int list[MAX_BATCH * 16];
  int wave_cnt[NWAVE];
  int ecnt[MAX_SHARE_EXPERTS];  // sequences routed to each expert (TF_SHARE)
  int ne[MAX_SHARE_EXPERTS];    // the experts with any, ascending
  int n_ne;
};
static_assert(sizeof(ExpLds) <= sizeof(float) * LDS_VEC + sizeof(uint4) * NWAVE * STAGE_CHUNKS * 64,
              "expert LDS exceeds the overlaid areas");

// One expert (a0), part q: for every sequence routed to it (in sequence,
// slot order, EXP_GROUP at a time), the gate/up rows a1 .. a1 + a2 with
// SwiGLU into the activation words of that (sequence, slot); then the down
// rows of the same expert over the full activations (from every part of the
// expert) into the expert-output words y of that (sequence, slot). Both are
// MFMA GEMMs with the group's inputs as the columns, so the time is the
// weights' streaming time whatever the number of routed sequences. Dense
// FFN: expert 0, every sequence in slot 0.
template <int CH, int TCH, int CF, int TCF>
__device__ __forceinline__ bool task_bexp(Ctx& c, const Task& t) {
  KAC& a = c.a;
  Smem& s = c.s;
  ExpLds& X = *(ExpLds*)&s;
  const int l = t.layer;
  const int H = a.H, F = a.F, KK = a.dense ? 1 : a.K, EE = a.dense ? 1 : a.E, B = a.B;
  const int th = tid(), lane = th & 63, w = th >> 6;
  const int n = B * KK;  // routed (sequence, slot) entries, <= NT (checked by the planner)
  if (!a.dense) {
    if (!gather_fn<1>(c, n, [&](int i) { return a.route + (size_t)l * a.s_route + (size_t)i * 2; }, X.ids, 0))
      return false;
  }
  // the routed list of expert e (entries b * KK + slot, ascending) into X.list; uniform count
  auto routed = [&](int e) -> int {
    if (a.dense) {
      for (int b = th; b < B; b += NT) X.list[b] = b;
      lds_barrier();
      return B;
    }
    const bool mine = th < n && __float_as_int(X.ids[th]) == e;
    const uint64_t m = __ballot(mine);
    if (lane == 0) X.wave_cnt[w] = __popcll(m);
    lds_barrier();
    int off = 0, ns = 0;
    for (int q = 0; q < w; ++q) off += X.wave_cnt[q];
    for (int q = 0; q < NWAVE; ++q) ns += X.wave_cnt[q];
    if (mine) X.list[off + __popcll(m & ((1ull << lane) - 1ull))] = th;
    lds_barrier();
    return ns;
  };
  Gains gn;
  gn.load(a.ffn_norm + (size_t)l * H, H);
  const int ldh = exp_ld(H), ldf = exp_ld(F);
  const int kq = lane >> 4, r16 = lane & 15;
  // gate/up rows of FFN rows f0 .. f0 + nf of expert e, for its routed sequences
  auto gateup = [&](int e, int f0, int nf) -> bool {
    const int ns = routed(e);
    if (ns == 0 || nf == 0) return true;
    const uint16_t* Wg = a.gate + ((size_t)l * EE + e) * F * H;
    const uint16_t* Wu = a.up + ((size_t)l * EE + e) * F * H;
    // rows 2f (gate) and 2f + 1 (up) of FFN row f0 + f
    for (int g0 = 0; g0 < ns; g0 += EXP_GROUP) {
      const int ng = min(EXP_GROUP, ns - g0);
      // column q at the padded stride
      // H is even (a multiple of 256 for batch plans): pairs stay in one column
      if (!gather_fn_pairs<4>(c, ng * H, [&](int i) {
            const int q = i / H, bs = X.list[g0 + q] / KK;
            return a.xa + (size_t)l * a.s_x + (size_t)bs * H + (i - q * H);
          }, X.in, 1, [&](int i) { const int q = i / H; return q * ldh + (i - q * H); }))
        return false;
      for (int q = 0; q < ng; ++q) rmsnorm_pack(c, X.in + (size_t)q * ldh, H, gn);
      // rows 2f (gate) and 2f + 1 (up) of FFN row f0 + f: from the tile copy
      // when there is one (its 16-row blocks start at FFN rows 8i), else row-major
      const bool tl = a.etile && (f0 & 7) == 0 && (nf & 7) == 0;
      const uint4* gt = tl ? (const uint4*)(a.etile + ((size_t)l * EE + e) * 3 * F * H) +
                                 (size_t)(f0 >> 3) * (H >> 5) * 64 + lane
                           : nullptr;
      mfma_rows(2 * nf, H, [&](int rb) -> const uint4* {
          if (tl) return gt + (size_t)rb * (H >> 5) * 64;
          const int j = min(rb * 16 + r16, 2 * nf - 1);
          return (const uint4*)(((j & 1) ? Wu : Wg) + (size_t)(f0 + (j >> 1)) * H + 8 * kq);
        }, tl ? 64 : 4, X.in, ldh, ng, [&](int rb, const v4f& acc) {
          // rows 16 rb + 4 kq + j: j = 0, 1 gate and up of one FFN row, j = 2, 3 of the next
          if (r16 < ng) {
            const int ent = X.list[g0 + r16];  // b * KK + slot
            uint64_t* dst = a.act + (size_t)l * a.s_act + (size_t)ent * F + f0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int f = (rb * 16 + 4 * kq + 2 * h) >> 1;
              const float yg = acc[2 * h], yu = acc[2 * h + 1];
              if (f < nf) st_tagged(dst + f, yg / (1.0f + expf(-yg)) * yu, a.epoch);
            }
          }
        });
      lds_barrier();
    }
    return true;
  };
  // down rows r0 .. r0 + nr of expert e over the full activations of each routed slot
  auto down = [&](int e, int r0, int nr) -> bool {
    const int ns = routed(e);
    if (ns == 0 || nr == 0) return true;
    const uint16_t* Wd = a.down + ((size_t)l * EE + e) * H * F;
    for (int g0 = 0; g0 < ns; g0 += EXP_GROUP) {
      const int ng = min(EXP_GROUP, ns - g0);
      for (int q = 0; q < ng; ++q)
        if (!gather_split<4>(c, a.act + (size_t)l * a.s_act + (size_t)X.list[g0 + q] * F, F,
                             X.in + (size_t)q * ldf, 1))
          return false;
      // hidden rows r0 + j: the tile copy's down part (16-row blocks from row 0) or row-major
      const bool tl = a.etile && (r0 & 15) == 0 && (nr & 15) == 0;
      const uint4* dt = tl ? (const uint4*)(a.etile + ((size_t)l * EE + e) * 3 * F * H + 2 * (size_t)F * H) +
                                 (size_t)(r0 >> 4) * (F >> 5) * 64 + lane
                           : nullptr;
      mfma_rows(nr, F, [&](int rb) -> const uint4* {
          if (tl) return dt + (size_t)rb * (F >> 5) * 64;
          return (const uint4*)(Wd + (size_t)(r0 + min(rb * 16 + r16, nr - 1)) * F + 8 * kq);
        }, tl ? 64 : 4, X.in, ldf, ng,
                [&](int rb, const v4f& acc) {
          if (r16 < ng) {
            const int ent = X.list[g0 + r16];
            uint64_t* dst = a.y + (size_t)l * a.s_y + (size_t)ent * H + r0;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int r = rb * 16 + 4 * kq + jj;
              if (r < nr) st_tagged(dst + r, acc[jj], a.epoch);
            }
          }
        });
      lds_barrier();
    }
    return true;
  };
  mark(c, 0);
  if (!(t.flags & TF_SHARE)) {
    // one expert (a0), part q: gate/up rows a1 .. a1 + a2, down rows a3
    const int e = t.a0, f0 = t.a1, nf = t.a2, r0 = t.a3 >> 16, nr = t.a3 & 0xFFFF;
    if (!gateup(e, f0, nf)) return false;
    mark(c, 1);
    if (!down(e, r0, nr)) return false;
    mark(c, 2);
    return true;
  }
  // Share aux of a1: list the experts any sequence chose (ascending), then
  // take rows [i T_g / a1, (i + 1) T_g / a1) of their concatenated gate/up
  // rows (8 FFN rows per unit) and likewise of their down rows (16 per unit)
  const int E = a.E;
  for (int i = th; i < E; i += NT) X.ecnt[i] = 0;
  lds_barrier();
  if (th < n) {
    const int id = __float_as_int(X.ids[th]);
    if (id >= 0 && id < E) atomicAdd(&X.ecnt[id], 1);
  }
  lds_barrier();
  if (w == 0) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const bool ne = e < E && X.ecnt[e] > 0;
      const uint64_t m = __ballot(ne);
      if (ne) X.ne[base + __popcll(m & ((1ull << lane) - 1ull))] = e;
      base += __popcll(m);
    }
    if (lane == 0) X.n_ne = base;
  }
  lds_barrier();
  const int n_ne = X.n_ne, T = t.a1, me = t.aux;
  {
    const int U = F / 8;
    const int64_t tot = (int64_t)n_ne * U;
    int64_t u = tot * me / T;
    const int64_t ub = tot * (me + 1) / T;
    while (u < ub) {
      const int i = (int)(u / U), fu = (int)(u % U);
      const int take = (int)min((int64_t)(U - fu), ub - u);
      if (!gateup(X.ne[i], 8 * fu, 8 * take)) return false;
      u += take;
    }
  }
  mark(c, 1);
  {
    const int U = H / 16;
    const int64_t tot = (int64_t)n_ne * U;
    int64_t u = tot * me / T;
    const int64_t ub = tot * (me + 1) / T;
    while (u < ub) {
      const int i = (int)(u / U), fu = (int)(u % U);
      const int take = (int)min((int64_t)(U - fu), ub - u);
      if (!down(X.ne[i], 16 * fu, 16 * take)) return false;
      u += take;
    }
  }
  mark(c, 2);
  return true;
}

// Hidden rows a1 .. a1 + a2 of sequence a0 after the FFN: the residual plus
// the routing-weighted sum of its experts' outputs, in slot order.
__device__ __forceinline__ bool task_bcomb(Ctx& c, const Task& t) {
  KAC& a = c.a;
  Smem& s = c.s;
  const int l = t.layer, b = t.a0, r0 = t.a1, nr = t.a2, H = a.H;
  const int KK = a.dense ? 1 : a.K;
  // words: [weights (KK, MoE only)] [y slot 0 rows] .. [y slot KK-1 rows] [residual rows]
  const int nw = a.dense ? 0 : KK;
  const int n = nw + (KK + 1) * nr;
  float* v = s.vec;
  if (!gather_fn<4>(c, n, [&](int i) -> const uint64_t* {
        if (i < nw) return a.route + (size_t)l * a.s_route + ((size_t)b * KK + i) * 2 + 1;
        i -= nw;
        const int j = i / nr, r = i - j * nr;
        if (j < KK) return a.y + (size_t)l * a.s_y + ((size_t)b * KK + j) * H + r0 + r;
        return a.xa + (size_t)l * a.s_x + (size_t)b * H + r0 + r;
      }, v, 1))
    return false;
  for (int r = tid(); r < nr; r += NT) {
    float y = 0.f;
    for (int j = 0; j < KK; ++j) y += (a.dense ? 1.f : v[j]) * v[nw + j * nr + r];
    st_tagged(a.x + (size_t)l * a.s_x + (size_t)b * H + r0 + r, v[nw + KK * nr + r] + y, a.epoch);
  }
  return true;
}

// LM-head rows for every sequence, then each sequence's argmax over them.
__device__ __forceinline__ bool task_blm(Ctx& c, const Task& t) {
  KAC& a = c.a;
  const int r0 = t.a1, n = t.a2, H = a.H, B = a.B;
  MtSrc src{a.x + (size_t)(a.L - 1) * a.s_x, H, a.final_norm, true};
  if (a.trace && tid() == 0) c.s.tw[2] = now();
  if (!mt_tile(c, n, H, [&](int j) { return a.lm + (size_t)(r0 + j) * H; }, src)) return false;
  if (a.trace && tid() == 0) c.s.tw[3] = now();
  const MtLds& P = *(const MtLds*)&c.s;
  // 16 threads per sequence
  const int b = tid() >> 4, sub = tid() & 15;
  float bv = NEG_INF;
  int bi = 0x7fffffff;
  if (b < B)
    for (int r = sub; r < n; r += 16) {
      const float y = P.out[r][b];
      if (a.logits) a.logits[(size_t)b * a.V + r0 + r] = y;
      if (a.smp_u) st_tagged(a.lw + (size_t)b * a.V + r0 + r, y, a.epoch);
      argmax_merge(y, r0 + r, bv, bi);
    }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_merge(ov, oi, bv, bi);
  }
  if (b < B && sub == 0) {
    uint64_t* dst = a.lmpart + ((size_t)t.a3 * B + b) * 2;
    st_tagged(dst, bv, a.epoch);
    st_tagged(dst + 1, __int_as_float(bi), a.epoch);
  }
  return true;
}

// Sequence a1's greedy token: the argmax over every LM-head tile's partial.
__device__ __forceinline__ bool task_bfinal(Ctx& c, const Task& t) {
  KAC& a = c.a;
  Smem& s = c.s;
  const int n = t.a0, b = t.a1, B = a.B;
  if (!gather_fn<2>(c, 2 * n, [&](int i) { return a.lmpart + ((size_t)(i >> 1) * B + b) * 2 + (i & 1); },
                    s.vec, 1))
    return false;
  float bv = NEG_INF;
  int bi = 0x7fffffff;
  for (int q = tid(); q < n; q += NT) argmax_merge(s.vec[2 * q], __float_as_int(s.vec[2 * q + 1]), bv, bi);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_merge(ov, oi, bv, bi);
  }
  float* rv = s.red;
  int* ri = (int*)(s.red + NWAVE);
  if ((tid() & 63) == 0) { rv[tid() >> 6] = bv; ri[tid() >> 6] = bi; }
  lds_barrier();
  if (sampling(a, b)) {
    int* tok = &s.tok;
    if (!sample_seq(c, b, n, t.a2, [&](int i) { return s.vec[2 * i]; },
                    [&](int i) { return __float_as_int(s.vec[2 * i + 1]); }, tok))
      return false;
    if (tid() == 0) {
      a.tok_out[b] = *tok;
      a.seq_lens[b] = a.seq_lens[b] + 1;
    }
    return true;
  }
  if (tid() == 0) {
    for (int q = 1; q < NWAVE; ++q) argmax_merge(rv[q], ri[q], bv, bi);
    a.tok_out[b] = bi;
    a.seq_lens[b] = a.seq_lens[b] + 1;
  }
  return true;
}

// One kernel per shape class: CH, CO, CF are the 16-byte chunks per lane of
// the GEMVs over the hidden size, the attention output (query heads x head
// dim) and the FFN width, TCH, TCO, TCF their lane-group widths; HD is the
// head dim. Each variant contains only the
// task bodies its shapes use, so registers are allocated for them alone.
template <int CH, int TCH, int CO, int TCO, int CF, int TCF, int HD, bool BATCH>
__global__ void __launch_bounds__(NT) megakernel(KArgs) {
  __shared__ Smem s;
  // explicit kernel arguments start at offset 0 of the kernel-argument segment
  const KAC* const args = (const KAC*)__builtin_amdgcn_kernarg_segment_ptr();
  const uint32_t* hdr = args->plan;
  const uint32_t* off = hdr + PLAN_HDR_WORDS;
  const Task* tasks = (const Task*)((const char*)hdr + hdr[H_TASK_OFF_BYTES]);
  const Task* splits = (const Task*)((const char*)hdr + hdr[H_SPLIT_OFF_BYTES]);  // queue plans
  const uint32_t beg = off[blockIdx.x], end = off[blockIdx.x + 1];
  if (tid() == 0) {
    s.fail = 0;
    s.kv_ti = -1;
  }
  lds_barrier();
  for (uint32_t ti = beg; ti < end; ++ti) {
    // an opaque copy of the argument pointer per task: fields are loaded where
    // a body uses them instead of being kept live across the loop
    const KAC* pa = args;
    asm volatile("" : "+s"(pa));
    KAC& a = *pa;
    const Task t = tasks[ti];
    Ctx c{a, s, now(), ti};
    if (a.trace && tid() == 0) {
      s.tw[0] = s.tw[1] = s.tw[2] = s.tw[3] = 0;
      for (int i = 0; i < TRACE_MARKS; ++i) s.mk[i] = 0;
    }
    bool ok = true;
    uint32_t units = t.units;  // outputs this task adds to its completion counter
    if (t.flags & TF_STAGE_KV) {
      // the first attention task further on in this unit's list (the planner
      // checked that there is one within STAGE_SCAN tasks)
      uint32_t ta = ti + 1;
      while (ta < end && ta <= ti + STAGE_SCAN && tasks[ta].op != OP_ATTN) ++ta;
      if (ta < end && ta <= ti + STAGE_SCAN) stage_kv<HD>(c, tasks[ta], ta);
    }
    switch (t.op) {
      case OP_ATTN: {
        // One split, or splits from the shared queue (records a1 .. a1 + a2
        // of the plan's split table, longest first): every pull adds one to
        // the queue counter; this step's pulls are numbered from base =
        // (epoch - 1) * (splits + queue tasks), since each queue task's last
        // pull comes back empty. The next split is pulled while one runs.
        const bool queue = (t.flags & TF_QUEUE) != 0;
        uint32_t* qc = a.ctr + (size_t)t.a0 * CTR_LINES * CTR_STRIDE;
        const uint32_t n_items = queue ? (uint32_t)t.a2 : 1u;
        const uint32_t base = (a.epoch - 1u) * (n_items + (uint32_t)t.a3);
        if (queue && tid() == 0)
          s.qnext = __hip_atomic_fetch_add(qc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - base;
        if (queue) lds_barrier();
        Task tt = t;
        while (true) {
          uint32_t nxt = 0;
          if (queue) {
            const uint32_t idx = s.qnext;
            if (idx >= n_items) break;
            lds_barrier();  // every wave has read qnext
            if (tid() == 0) nxt = __hip_atomic_fetch_add(qc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            tt = splits[t.a1 + idx];
            tt.layer = t.layer;
          }
          ok = task_attn<HD>(c, tt);
          if (queue) units += (uint32_t)tt.a3;  // a pulled split adds its pages
          if (!ok || !queue) break;
          if (tid() == 0) s.qnext = nxt - base;
          lds_barrier();
        }
        break;
      }
      case OP_COMB: ok = task_comb<BATCH>(c, t); break;
      default:
        if constexpr (BATCH) {
          switch (t.op) {
            case OP_BQKV: ok = task_bqkv(c, t); break;
            case OP_BO: ok = task_bo(c, t); break;
            case OP_ROUTER: ok = task_router<CH, TCH>(c, t); break;
            case OP_TOPK: ok = task_topk<CH, TCH>(c, t); break;
            case OP_BEXP: ok = task_bexp<CH, TCH, CF, TCF>(c, t); break;
            case OP_BCOMB: ok = task_bcomb(c, t); break;
            case OP_BLM: ok = task_blm(c, t); break;
            case OP_BFINAL: ok = task_bfinal(c, t); break;
            default: break;
          }
        } else {
          switch (t.op) {
            case OP_QKV: ok = task_qkv<CH, TCH, HD>(c, t); break;
            case OP_O: ok = task_o<CO, TCO>(c, t); break;
            case OP_ROUTER:
              ok = (t.flags & TF_FOLD) ? task_router_fold(c, t) : task_router<CH, TCH>(c, t);
              break;
            case OP_EXPERT: ok = task_expert<CH, TCH, CF, TCF>(c, t); break;
            case OP_LM: ok = task_lm<CH, TCH>(c, t); break;
            case OP_FINAL: ok = task_final(c, t); break;
            default: break;
          }
        }
        break;
    }
    // A failure (recorded in the status words) may reach only some threads
    // (a residual wait in one lane): it is shared through LDS, so that the
    // whole workgroup leaves together.
    if (!ok) s.fail = 1;
    const uint64_t t_body = (a.trace && tid() == 0) ? now() : 0;
    lds_barrier();  // LDS is reused by the next task
    if (s.fail) return;
    if (tid() == 0) {
      if (t.signal != NO_CTR)
        __hip_atomic_fetch_add(a.ctr + ((size_t)t.signal * CTR_LINES + blockIdx.x % CTR_LINES) * CTR_STRIDE,
                               units, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.trace) {
        uint64_t* tr = a.trace + (size_t)ti * TRACE_WORDS;
        tr[0] = c.t0;
        tr[1] = s.tw[0]; tr[2] = s.tw[1]; tr[3] = s.tw[2]; tr[4] = s.tw[3];
        tr[5] = t_body;
        tr[6] = now();
        tr[7] = ((uint64_t)blockIdx.x << 32) | ((uint64_t)t.op << 16) | t.layer;
        for (int i = 0; i < TRACE_MARKS; ++i) tr[8 + i] = s.mk[i];
      }
    }
  }
}


// Streaming copy with the 16-byte non-temporal loads the task bodies use for
// weights: the bandwidth probe behind the roofline's achievable ceiling and
// the known-size kernel that calibrates hardware byte counters.
__global__ __launch_bounds__(256) void mk_stream_copy_kernel(uint4* __restrict__ dst,
                                                             const uint4* __restrict__ src, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 v = ld_nt(src + i);
    __builtin_nontemporal_store(u4v{v.x, v.y, v.z, v.w}, (u4v*)(dst + i));
  }
}

// out[l][e][j] = sum_h R[l][e][h] g[l][h] O[l][h][j] (mk_router_fold): a
// 32 (e) x 64 (j) tile per workgroup of 256 threads, 2 x 4 outputs per
// thread, h in LDS-staged steps of 32. Each term is a product of three bf16
// values (at most 24 significant bits), exact in fp32; sums in fp32.
__global__ __launch_bounds__(256) void mk_router_fold_kernel(const uint16_t* __restrict__ R,
                                                             const uint16_t* __restrict__ g,
                                                             const uint16_t* __restrict__ O,
                                                             float* __restrict__ out, int E, int H, int K) {
  __shared__ float As[32][33];
  __shared__ float Bs[32][64];
  const int l = blockIdx.z, e0 = blockIdx.y * 32, j0 = blockIdx.x * 64;
  const int te = threadIdx.x / 16, tj = threadIdx.x % 16;
  const size_t ld = (size_t)H + K;  // output row: [R diag(g) (H) | R diag(g) O (K)]
  const uint16_t* Rl = R + (size_t)l * E * H;
  const uint16_t* gl = g + (size_t)l * H;
  const uint16_t* Ol = O + (size_t)l * H * K;
  float acc[2][4] = {};
  for (int h0 = 0; h0 < H; h0 += 32) {
    for (int i = threadIdx.x; i < 32 * 32; i += 256) {
      const int e = i / 32, h = i % 32;
      As[e][h] = e0 + e < E && h0 + h < H ? bf2f(Rl[(size_t)(e0 + e) * H + h0 + h]) * bf2f(gl[h0 + h]) : 0.f;
    }
    for (int i = threadIdx.x; i < 32 * 64; i += 256) {
      const int h = i / 64, j = i % 64;
      Bs[h][j] = h0 + h < H && j0 + j < K ? bf2f(Ol[(size_t)(h0 + h) * K + j0 + j]) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int h = 0; h < 32; ++h) {
      const float a0 = As[2 * te][h], a1 = As[2 * te + 1][h];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float bv = Bs[h][4 * tj + q];
        acc[0][q] = fmaf(a0, bv, acc[0][q]);
        acc[1][q] = fmaf(a1, bv, acc[1][q]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + 2 * te + r, j = j0 + 4 * tj + q;
      if (e < E && j < K) out[((size_t)l * E + e) * ld + H + j] = acc[r][q];
    }
}

// The first H columns of mk_router_fold's rows: R[l][e][h] g[l][h] (exact in fp32).
__global__ __launch_bounds__(256) void mk_router_scale_kernel(const uint16_t* __restrict__ R,
                                                              const uint16_t* __restrict__ g,
                                                              float* __restrict__ out, int L, int E, int H, int K) {
  const size_t n = (size_t)L * E * H, stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const size_t h = i % H, le = i / H, l = le / E;
    out[le * ((size_t)H + K) + h] = bf2f(R[i]) * bf2f(g[l * H + h]);
  }
}

// Zero-fill of n 16-byte words (a kernel, not a memset node, so that a
// caller may capture it in a graph).
// Expert weights in MFMA tile order (mk_expert_tile). Per layer l and
// expert e, 3 F H bf16: the gate/up rows (row 2f = gate row f, 2f + 1 = up
// row f) as 2F/16 row blocks, then the down rows as H/16 row blocks; a row
// block of K columns is K/32 tiles of 64 x 16 bytes, lane t holding the 8
// values of row 16 rb + t % 16 at columns 32 s + 8 (t / 16) .. + 7: the
// A operand of v_mfma_f32_16x16x32_bf16 for k-step s, one kilobyte per wave
// load. One uint4 per thread, grid-stride.
__global__ __launch_bounds__(256) void mk_expert_tile_kernel(const uint16_t* __restrict__ gate,
                                                             const uint16_t* __restrict__ up,
                                                             const uint16_t* __restrict__ down,
                                                             uint4* __restrict__ out, int LE, int H, int F) {
  const size_t per = (size_t)3 * F * H / 8;  // uint4 per (layer, expert)
  const size_t gu = (size_t)2 * F * H / 8;
  const size_t n = per * (size_t)LE;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t le = i / per, q = i - le * per;
    const int lane = (int)(q & 63);
    const size_t t = q >> 6;  // tile index within the part
    const uint16_t* src;
    if (q < gu) {
      const int ks = H >> 5;
      const size_t rb = t / ks, st = t - rb * ks;
      const size_t j = rb * 16 + (lane & 15);  // interleaved gate/up row
      src = ((j & 1) ? up : gate) + (le * F + (j >> 1)) * H + st * 32 + 8 * (lane >> 4);
    } else {
      const int ks = F >> 5;
      const size_t t2 = t - gu / 64;
      const size_t rb = t2 / ks, st = t2 - rb * ks;
      const size_t r = rb * 16 + (lane & 15);
      src = down + (le * H + r) * F + st * 32 + 8 * (lane >> 4);
    }
    out[i] = *(const uint4*)src;
  }
}

__global__ __launch_bounds__(256) void mk_zero_kernel(uint4* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

// Kernel variants, indexed by mk::kernel_class (see mk_internal.hpp) and by
// batch (batch 1: GEMV tiles; a batch: MFMA tiles and shared expert tasks).
const void* kernel_for(int cls, bool batch) {
  switch (cls * 2 + (batch ? 1 : 0)) {
    case 0: return (const void*)megakernel<1, 32, 1, 32, 1, 64, 64, false>;   // hidden 256, 4x64 heads, FFN 512
    case 1: return (const void*)megakernel<1, 32, 1, 32, 1, 64, 64, true>;
    case 2: return (const void*)megakernel<2, 64, 2, 64, 1, 64, 64, false>;   // hidden 1024, 16x64 heads, FFN 512
    case 3: return (const void*)megakernel<2, 64, 2, 64, 1, 64, 64, true>;
    case 4: return (const void*)megakernel<4, 64, 8, 64, 3, 32, 128, false>;  // hidden 2048, 32x128 heads, FFN 768
    case 5: return (const void*)megakernel<4, 64, 8, 64, 3, 32, 128, true>;
    default: return nullptr;
  }
}

}  // namespace dev
}  // namespace mk

// ------------------------------------------------------------------ host side

using mkh::fail;

static mk_status hip_fail(hipError_t e, const char* what) {
  return fail(MK_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

extern "C" mk_status mk_device_cu_count(int32_t* n_cu) {
  if (!n_cu) return fail(MK_EINVAL, "mk_device_cu_count: NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  *n_cu = v;
  return MK_OK;
}

extern "C" mk_status mk_expert_tile(const mk_model_desc* m, const mk_weights* w, void* out, void* stream) {
  if (!m || !w || !out) return fail(MK_EINVAL, "mk_expert_tile: NULL argument");
  if (!w->gate || !w->up || !w->down) return fail(MK_EINVAL, "mk_expert_tile: missing weight pointer");
  const bool moe = m->n_experts > 0;
  const int L = m->n_layers, H = m->hidden, E = moe ? m->n_experts : 1, F = moe ? m->expert_ffn : m->ffn_dim;
  if (L <= 0 || H <= 0 || F <= 0 || E <= 0) return fail(MK_EINVAL, "mk_expert_tile: bad shape");
  if (H % 32 || F % 32) return fail(MK_EUNSUPPORTED, "mk_expert_tile: hidden and FFN widths must be multiples of 32");
  if (((uintptr_t)out | (uintptr_t)w->gate | (uintptr_t)w->up | (uintptr_t)w->down) & 15)
    return fail(MK_EINVAL, "mk_expert_tile: pointers must be 16-byte aligned");
  hipLaunchKernelGGL(mk::dev::mk_expert_tile_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)w->gate, (const uint16_t*)w->up, (const uint16_t*)w->down, (uint4*)out,
                     L * E, H, F);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "mk_expert_tile");
  return MK_OK;
}

extern "C" mk_status mk_router_fold(const mk_model_desc* m, const mk_weights* w, float* out, void* stream) {
  if (!m || !w || !out) return fail(MK_EINVAL, "mk_router_fold: NULL argument");
  if (m->n_experts <= 0) return fail(MK_EINVAL, "mk_router_fold: a dense model has no router");
  if (!w->router || !w->ffn_norm || !w->w_o) return fail(MK_EINVAL, "mk_router_fold: missing weight pointer");
  const int E = m->n_experts, H = m->hidden, K = m->n_q_heads * m->head_dim, L = m->n_layers;
  if (E <= 0 || H <= 0 || K <= 0 || L <= 0) return fail(MK_EINVAL, "mk_router_fold: bad shape");
  if ((H + K) % 4 || H + K > mk::dev::LDS_VEC)
    return fail(MK_EUNSUPPORTED, "mk_router_fold: hidden + heads x dim must be a multiple of 4, at most 8192");
  hipLaunchKernelGGL(mk::dev::mk_router_scale_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)w->router, (const uint16_t*)w->ffn_norm, out, L, E, H, K);
  hipLaunchKernelGGL(mk::dev::mk_router_fold_kernel, dim3((K + 63) / 64, (E + 31) / 32, L), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)w->router, (const uint16_t*)w->ffn_norm,
                     (const uint16_t*)w->w_o, out, E, H, K);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "mk_router_fold");
  return MK_OK;
}

extern "C" mk_status mk_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src) return fail(MK_EINVAL, "mk_stream_copy: NULL pointer");
  if (bytes % 16 || ((uintptr_t)dst | (uintptr_t)src) % 16)
    return fail(MK_EINVAL, "mk_stream_copy: bytes and both pointers must be multiples of 16");
  if (bytes == 0) return MK_OK;
  const size_t n = bytes / 16;
  int32_t cus = 0;
  mk_status st = mk_device_cu_count(&cus);
  if (st != MK_OK) return st;
  const size_t want = (n + 255) / 256;
  const unsigned grid = (unsigned)std::min<size_t>(want, (size_t)cus * 16);
  hipLaunchKernelGGL(mk::dev::mk_stream_copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (uint4*)dst, (const uint4*)src, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "mk_stream_copy launch");
  return MK_OK;
}

extern "C" mk_status mk_plan_upload(const mk_plan_t* p, void* d_plan, size_t bytes, void* stream) {
  if (!p || !d_plan) return fail(MK_EINVAL, "mk_plan_upload: NULL argument");
  if (bytes < p->image.size()) return fail(MK_EINVAL, "mk_plan_upload: device buffer too small");
  hipError_t e = hipMemcpyAsync(d_plan, p->image.data(), p->image.size(), hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  e = hipStreamSynchronize((hipStream_t)stream);  // the host image may be freed with the plan
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(plan)");
  return MK_OK;
}

extern "C" mk_status mk_step_status(const uint32_t* h) {
  if (!h) return fail(MK_EINVAL, "mk_step_status: NULL");
  switch (h[0]) {
    case mk::DS_OK: return MK_OK;
    case mk::DS_TIMEOUT: {
      // word 3 tells the kind of wait: a gather of word pairs, a batch
      // activation panel, or a single word (then word 3 is the tag it held)
      const std::string what = h[3] == 0xFFFFFFFDu   ? "gather of word pairs (stale pair " + std::to_string(h[2]) + ")"
                               : h[3] == 0xFFFFFFFEu ? "activation panel of sequence " + std::to_string(h[2])
                                                     : "buffer word " + std::to_string(h[2]) + " tag seen " +
                                                           std::to_string(h[3]);
      return fail(MK_ETIMEOUT, "device wait timed out: task " + std::to_string(h[1]) + ", " + what);
    }
    case mk::DS_BOUNDS:
      return fail(MK_EBOUNDS, "device bounds check failed: task " + std::to_string(h[1]) +
                                  " (token, position or page outside the plan/pool)");
    default:
      return fail(MK_EDEVICE, "unknown device status " + std::to_string(h[0]));
  }
}

// One step of plan p with the step buffers bu (checked by the caller).
static mk_status launch_step(const mk_plan_t* p, const mk_weights* w, const mk_kv* kv, const mk_io* io,
                             const mk_step_buffers* bu, uint32_t epoch, uint32_t timeout_ms, void* stream);

extern "C" mk_status mk_decode_step(const mk_plan_t* p, const mk_weights* w, const mk_kv* kv,
                                    const mk_io* io, const mk_step_buffers* bu, uint32_t epoch,
                                    uint32_t timeout_ms, void* stream) {
  if (!p || !w || !kv || !io || !bu) return fail(MK_EINVAL, "mk_decode_step: NULL argument");
  if (!bu->plan || bu->plan_bytes < p->image.size() || !bu->workspace ||
      bu->workspace_bytes < p->ws_total || !bu->counters ||
      bu->counter_bytes < p->targets.size() * mk::CTR_LINES * mk::CTR_STRIDE * 4 || !bu->status)
    return fail(MK_EINVAL, "mk_decode_step: step buffers missing or too small");
  return launch_step(p, w, kv, io, bu, epoch, timeout_ms, stream);
}

// ------------------------------------------------------------------ static scratch
//
// The allocation-free step keeps the workspace (tagged activations) and the
// completion counters of its plan in this file-scope array instead of caller
// buffers. Each device holds its own copy; its address on the current device
// is looked up once per device with hipGetSymbolAddress and used wherever the
// host needs the array's memory (the array's name in host code is not a
// device address).
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)MK_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

namespace {
struct StaticState {
  uint8_t* ptr = nullptr;  // the device address of scratch on this device
  uint64_t plan_uid = 0;   // plan whose workspace the scratch holds (0: none)
  uint32_t epoch = 0;      // last epoch used on it
};
std::mutex g_static_mu;
std::map<int, StaticState> g_static;  // per device
}  // namespace

extern "C" mk_status mk_decode_step_static(const mk_plan_t* p, const mk_weights* w, const mk_kv* kv,
                                           const mk_io* io, const void* d_plan, size_t plan_bytes,
                                           uint32_t* d_status, uint32_t timeout_ms, void* stream) {
  if (!p || !w || !kv || !io || !d_plan || !d_status)
    return fail(MK_EINVAL, "mk_decode_step_static: NULL argument");
  if (plan_bytes < p->image.size()) return fail(MK_EINVAL, "mk_decode_step_static: plan buffer too small");
  const size_t ws = (p->ws_total + 255) & ~(size_t)255;
  const size_t ctr = p->targets.size() * mk::CTR_LINES * mk::CTR_STRIDE * 4;
  if (ws + ctr > STATIC_SCRATCH_BYTES)
    return fail(MK_EBOUNDS, "mk_decode_step_static: the plan needs " + std::to_string(ws + ctr) +
                                " bytes of workspace and counters; the static scratch holds " +
                                std::to_string(STATIC_SCRATCH_BYTES) + " (use mk_decode_step)");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  uint8_t* base = nullptr;
  uint32_t epoch = 0;
  bool clear = false;
  {
    std::lock_guard<std::mutex> lk(g_static_mu);
    StaticState& st = g_static[dev];
    if (!st.ptr) {
      e = hipGetSymbolAddress((void**)&st.ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        st.ptr = nullptr;
        return hip_fail(e, "hipGetSymbolAddress(scratch)");
      }
    }
    // a plan other than the last one on this device: its workspace and
    // counters start from zero and its epochs from 1
    if (st.plan_uid != p->uid) {
      st.plan_uid = p->uid;
      st.epoch = 0;
      clear = true;
    }
    if (st.epoch == 0xFFFFFFFFu) return fail(MK_ESTATE, "mk_decode_step_static: epochs of this plan exhausted");
    epoch = ++st.epoch;
    base = st.ptr;
  }
  if (clear) {
    const size_t n = (ws + ctr) / 16;
    int32_t cus = 0;
    mk_status sc = mk_device_cu_count(&cus);
    if (sc != MK_OK) return sc;
    const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, (size_t)cus * 8);
    hipLaunchKernelGGL(mk::dev::mk_zero_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (uint4*)base, n);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "mk_decode_step_static: zero-fill launch");
  }
  mk_step_buffers bu;
  std::memset(&bu, 0, sizeof bu);
  bu.plan = d_plan;
  bu.plan_bytes = plan_bytes;
  bu.workspace = base;
  bu.workspace_bytes = ws;
  bu.counters = (uint32_t*)(base + ws);
  bu.counter_bytes = ctr;
  bu.status = d_status;
  return launch_step(p, w, kv, io, &bu, epoch, timeout_ms, stream);
}

static mk_status launch_step(const mk_plan_t* p, const mk_weights* w, const mk_kv* kv, const mk_io* io,
                             const mk_step_buffers* bu, uint32_t epoch, uint32_t timeout_ms, void* stream) {
  const auto& m = p->m;
  const bool moe = m.n_experts > 0;
  if (!w->embed || !w->attn_norm || !w->w_qkv || !w->w_o || !w->ffn_norm || !w->gate || !w->up ||
      !w->down || !w->final_norm || !w->lm_head || (moe && !w->router))
    return fail(MK_EINVAL, "mk_decode_step: missing weight pointer");
  if (!kv->pool || !kv->page_table || !kv->seq_lens || !kv->rope_cos || !kv->rope_sin)
    return fail(MK_EINVAL, "mk_decode_step: missing KV pointer");
  if (kv->n_rope_pos < p->bound)
    return fail(MK_EBOUNDS, "mk_decode_step: rotary tables cover fewer positions than the plan bound");
  if (kv->n_pages <= 0) return fail(MK_EINVAL, "mk_decode_step: empty KV pool");
  if (!io->tokens_in || !io->tokens_out) return fail(MK_EINVAL, "mk_decode_step: missing token buffers");
  if (epoch == 0) return fail(MK_EINVAL, "mk_decode_step: epoch must be >= 1");

  mk::KArgs a;
  std::memset(&a, 0, sizeof a);
  a.L = m.n_layers; a.H = m.hidden; a.Hq = m.n_q_heads; a.Hkv = m.n_kv_heads; a.D = m.head_dim;
  a.HG = p->HG; a.F = p->F; a.E = moe ? m.n_experts : 1; a.K = moe ? m.top_k : 1;
  a.V = m.vocab; a.B = p->B; a.max_pages = p->max_pages; a.dense = moe ? 0 : 1;
  a.norm_topk = m.norm_topk; a.eps = m.rms_eps; a.attn_scale = (float)(1.0 / std::sqrt((double)a.D));
  a.embed = (const uint16_t*)w->embed; a.attn_norm = (const uint16_t*)w->attn_norm;
  a.wqkv = (const uint16_t*)w->w_qkv; a.wo = (const uint16_t*)w->w_o;
  a.ffn_norm = (const uint16_t*)w->ffn_norm; a.router = (const uint16_t*)w->router;
  a.gate = (const uint16_t*)w->gate; a.up = (const uint16_t*)w->up; a.down = (const uint16_t*)w->down;
  a.final_norm = (const uint16_t*)w->final_norm; a.lm = (const uint16_t*)w->lm_head;
  a.rfold = w->router_fold;
  a.etile = (const uint16_t*)w->expert_tiles;
  if (a.etile && ((uintptr_t)a.etile & 15))
    return fail(MK_EINVAL, "mk_decode_step: expert tiles not 16-byte aligned");
  if (p->router_fold && !w->router_fold)
    return fail(MK_EINVAL, "mk_decode_step: this plan reads the folded router (mk_router_fold) and it is NULL");
  a.pool = (uint16_t*)kv->pool;
  a.layer_stride = (int64_t)m.n_kv_heads * 2 * 16 * m.head_dim;
  a.page_stride = (int64_t)m.n_layers * a.layer_stride;
  a.n_pages = kv->n_pages; a.page_table = kv->page_table; a.seq_lens = kv->seq_lens;
  a.rope_cos = kv->rope_cos; a.rope_sin = kv->rope_sin; a.n_rope = kv->n_rope_pos; a.bound = p->bound;
  a.tok_in = io->tokens_in; a.tok_out = io->tokens_out; a.topk_ids = io->topk_ids;
  a.topk_w = io->topk_w; a.logits = io->logits;
  char* ws = (char*)bu->workspace;
  if (p->ws_total >= (1ull << 32))
    return fail(MK_EUNSUPPORTED, "mk_decode_step: workspace of 4 GiB or more");
  if ((uintptr_t)ws & 255) return fail(MK_EINVAL, "mk_decode_step: workspace not 256-byte aligned");
  a.ws = (const uint64_t*)ws;
  a.ws_bytes = (uint32_t)p->ws_total;
  auto buf = [&](int which) { return (uint64_t*)(ws + p->ws_off[which]); };
  auto words = [&](int which) { return (int64_t)(p->ws_stride[which] / 8); };
  a.x = buf(MK_BUF_XFFN); a.xa = buf(MK_BUF_XATTN); a.q = buf(MK_BUF_Q); a.kvn = buf(MK_BUF_KVN);
  a.part = buf(MK_BUF_PART); a.o = buf(MK_BUF_O); a.rlog = buf(MK_BUF_RLOG); a.act = buf(MK_BUF_ACT);
  a.lmpart = buf(MK_BUF_LMPART); a.route = buf(MK_BUF_ROUTE); a.y = buf(MK_BUF_Y);
  a.opart = buf(MK_BUF_OPART); a.s_opart = words(MK_BUF_OPART);
  a.qpart = buf(MK_BUF_QPART); a.s_qpart = words(MK_BUF_QPART);
  a.lw = buf(MK_BUF_LOGIT);
  if (io->sampling) {
    const mk_sampling* sm = io->sampling;
    if (!sm->temperature || !sm->top_k || !sm->top_p || !sm->min_p || !sm->uniform)
      return fail(MK_EINVAL, "mk_decode_step: a sampling array is NULL");
    a.smp_t = sm->temperature; a.smp_k = sm->top_k; a.smp_p = sm->top_p; a.smp_minp = sm->min_p;
    a.smp_u = sm->uniform;
  }
  a.s_x = words(MK_BUF_XFFN); a.s_q = words(MK_BUF_Q); a.s_kvn = words(MK_BUF_KVN);
  a.s_part = words(MK_BUF_PART); a.s_o = words(MK_BUF_O); a.s_rlog = words(MK_BUF_RLOG);
  a.s_act = words(MK_BUF_ACT); a.s_route = words(MK_BUF_ROUTE); a.s_y = words(MK_BUF_Y);
  a.seq_bound = (const int32_t*)((const char*)bu->plan +
                                 reinterpret_cast<const uint32_t*>(p->image.data())[mk::H_BOUND_OFF_BYTES]);
  a.S_max = p->S_max; a.n_lm = p->n_lm;
  a.plan = (const uint32_t*)bu->plan; a.ctr = bu->counters; a.status = bu->status; a.epoch = epoch;
  a.timeout_ticks = (uint64_t)(timeout_ms ? timeout_ms : 2000) * 100000ull;
  if (bu->trace) {
    if (bu->trace_bytes < p->n_tasks * mk::TRACE_WORDS * sizeof(uint64_t))
      return fail(MK_EINVAL, "mk_decode_step: trace buffer smaller than 128 bytes per task");
    a.trace = bu->trace;
  }

  const void* kern = mk::dev::kernel_for(p->kernel_class, p->batch);
  if (!kern) return fail(MK_EUNSUPPORTED, "mk_decode_step: no kernel variant for this model shape");
  void* args[] = {&a};
  hipError_t e = hipLaunchCooperativeKernel(kern, dim3(p->n_cu), dim3(mk::NT), args, 0,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipLaunchCooperativeKernel(megakernel)");
  return MK_OK;
}
