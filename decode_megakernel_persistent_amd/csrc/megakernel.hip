// The persistent decode megakernel for gfx950 and its launch.
//
// One workgroup of 512 threads per compute unit walks its own task list
// (megakernel page, "What is a Megakernel?": one resident block per
// processor, work read from a task list in global memory, dependencies as
// counters in global memory that finished tasks increment and waiting tasks
// spin on). Every task first issues the loads that do not depend on other
// tasks (weights, KV of earlier steps), then waits for its producers, then
// computes, stores and signals.
//
// Task bodies:
//  - projections (QKV, O, router, expert gate/up, expert down, LM head) are
//    block GEMVs streaming 16-byte bf16 chunks per thread with fp32
//    accumulation and wave reductions; RMSNorm is recomputed as a prologue
//    by every consumer tile; RoPE + KV append, residual adds, SwiGLU, the
//    weighted expert combine and the local argmax are epilogues;
//  - paged attention splits use MFMA 16x16x16 bf16 tiles on 16-token pages
//    (queries and probabilities carried as bf16 hi + lo pairs), with an
//    online softmax across pages and a log-sum-exp merge across waves;
//  - the split combine is a log-sum-exp merge in fixed split order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>

#include "mk.h"
#include "mk_device.hpp"
#include "mk_internal.hpp"
#include "mk_plan.hpp"

namespace mk {
namespace dev {

constexpr int SMEM_MAIN = GEMV_LDS_FLOATS;   // per-row partial sums, attention merge
constexpr int SMEM_AUX = 4096;               // small reductions, routing, combine weights
constexpr float NEG_INF = -__builtin_inff();

struct Smem {
  float main[SMEM_MAIN];
  float aux[SMEM_AUX];
  int route_ids[16];
  float route_w[16];
  int flag;
  uint64_t tw[4];  // trace: (begin, end) of the routing wait and of the data wait
};

// ------------------------------------------------------------------ block GEMV

// Threads per row of a GEMV task, carried in the task record (high nibble of
// flags = log2 TC) so that index math derived from it is recomputed per task.
__device__ __forceinline__ int task_tc(const Task& t) { return 1 << (t.flags >> 4); }

// Jobs j < nj are rows; thread (rg = tid / TC, tc = tid % TC) takes jobs
// rg + k*TR, reading CPL 16-byte chunks (chunk index tc + c*TC) of each row and
// dotting them with its slice u[CPL*8] of the input vector. Rows move through
// two register batches of NR rows; both batches are issued before `ready`
// (the dependency wait, which also fills u). The reduced dot of job j is
// sum_s part[s*nj + j] over s < max(1, TC/64) after the final barrier.
template <int CPL, int NR, class RowFn, class ReadyFn>
__device__ __forceinline__ bool gemv_block(int nj, int TC, const RowFn& rowptr,
                                           const ReadyFn& ready, float* part, float* u) {
  const int tid = threadIdx.x;
  const int TR = NT / TC;
  const int rg = tid / TC, tc = tid % TC;
  const int my = rg < nj ? (nj - rg + TR - 1) / TR : 0;
  const int nb = (my + NR - 1) / NR;
  uint4 wa[NR][CPL], wb[NR][CPL];
  auto issue = [&](uint4 (&w)[NR][CPL], int bi) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int k = bi * NR + r;
      if (k < my) {
        const uint4* p = rowptr(rg + k * TR);
#pragma unroll
        for (int c = 0; c < CPL; ++c) w[r][c] = ld_nt(p + tc + c * TC);
      }
    }
  };
  auto consume = [&](uint4 (&w)[NR][CPL], int bi) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int k = bi * NR + r;
      if (k < my) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) s += dot8(w[r][c], u + c * 8);
        const int j = rg + k * TR;
        if (TC >= 64) {
          s = wave_sum(s);
          if ((tid & 63) == 0) part[(tc >> 6) * nj + j] = s;
        } else {
          s = group_sum(s, 32);
          if ((tid & 31) == 0) part[j] = s;
        }
      }
    }
  };
  issue(wa, 0);
  issue(wb, 1);
  if (!ready()) return false;
  for (int bi = 0; bi < nb; bi += 2) {
    consume(wa, bi);
    issue(wa, bi + 2);
    if (bi + 1 < nb) {
      consume(wb, bi + 1);
      issue(wb, bi + 3);
    }
  }
  __syncthreads();
  return true;
}

__device__ __forceinline__ float job_sum(const float* part, int nj, int TC, int j) {
  float s = part[j];
  for (int q = 1; q < TC / 64; ++q) s += part[q * nj + j];
  return s;
}

// Load this thread's slice of a K-vector (fp32 or bf16 source), optionally
// RMS-normalised with gains `gain`: u = x / sqrt(mean(x^2) + eps) * gain.
template <int CPL>
__device__ __forceinline__ void load_slice(const KArgs& a, const float* xf, const uint16_t* xb,
                                           const uint16_t* gain, int K, int TC, float* u,
                                           float* red8) {
  const int tc = threadIdx.x % TC;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = (tc + c * TC) * 8;
    if (xf) {
      const float4 p0 = *(const float4*)(xf + col);
      const float4 p1 = *(const float4*)(xf + col + 4);
      u[c * 8 + 0] = p0.x; u[c * 8 + 1] = p0.y; u[c * 8 + 2] = p0.z; u[c * 8 + 3] = p0.w;
      u[c * 8 + 4] = p1.x; u[c * 8 + 5] = p1.y; u[c * 8 + 6] = p1.z; u[c * 8 + 7] = p1.w;
    } else {
      const uint4 w = *(const uint4*)(xb + col);
      u[c * 8 + 0] = bf_lo(w.x); u[c * 8 + 1] = bf_hi(w.x);
      u[c * 8 + 2] = bf_lo(w.y); u[c * 8 + 3] = bf_hi(w.y);
      u[c * 8 + 4] = bf_lo(w.z); u[c * 8 + 5] = bf_hi(w.z);
      u[c * 8 + 6] = bf_lo(w.w); u[c * 8 + 7] = bf_hi(w.w);
    }
  }
  if (!gain) return;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL * 8; ++i) ss = fmaf(u[i], u[i], ss);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) tot += red8[w];
  tot *= (float)TC / (float)NT;  // every row group holds a full copy of the columns
  const float rs = 1.0f / sqrtf(tot / (float)K + a.eps);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int col = (tc + c * TC) * 8;
    const uint4 g = *(const uint4*)(gain + col);
    const float gv[8] = {bf_lo(g.x), bf_hi(g.x), bf_lo(g.y), bf_hi(g.y),
                         bf_lo(g.z), bf_hi(g.z), bf_lo(g.w), bf_hi(g.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) u[c * 8 + i] = u[c * 8 + i] * rs * gv[i];
  }
}

// Hidden state entering layer l (batch row 0): the embedding row for l = 0.
__device__ __forceinline__ void layer_input(const KArgs& a, int l, const float** xf,
                                            const uint16_t** xb) {
  if (l == 0) {
    int tok = a.tok_in[0];
    if (tok < 0 || tok >= a.V) {  // an id outside the vocabulary reads row 0 and is reported
      if (threadIdx.x == 0) raise_status(a, DS_BOUNDS, 0xFFFFFFFFu, (uint32_t)tok, 0u);
      tok = 0;
    }
    *xf = nullptr;
    *xb = a.embed + (size_t)tok * a.H;
  } else {
    *xf = a.xf + (size_t)(l - 1) * a.s_x;
    *xb = nullptr;
  }
}

// ------------------------------------------------------------------ routing

// softmax over the E router logits of layer l, top-k (ties to the lower
// index), weights renormalised over the selection when norm_topk. Wave 0
// computes; the result is in s.route_ids / s.route_w after the barrier.
__device__ __forceinline__ void route(const KArgs& a, int l, Smem& s) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const float* r = a.rlog + (size_t)l * a.s_rlog;
    float v[4];
    float mx = NEG_INF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < a.E ? r[e] : NEG_INF;
      mx = fmaxf(mx, v[i]);
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (lane + 64 * i) < a.E ? expf(v[i] - mx) : 0.f;
      sum += v[i];
    }
    sum = wave_sum(sum);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = (lane + 64 * i) < a.E ? v[i] / sum : NEG_INF;
    float wsum = 0.f;
    for (int j = 0; j < a.K; ++j) {
      float bv = NEG_INF;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p[i] > bv) { bv = p[i]; bi = lane + 64 * i; }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (lane == 0) { s.route_ids[j] = bi; s.route_w[j] = bv; }
      wsum += bv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == bi) p[i] = NEG_INF;
    }
    if (lane == 0 && a.norm_topk)
      for (int j = 0; j < a.K; ++j) s.route_w[j] = s.route_w[j] / wsum;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ tasks

template <int CPL>
__device__ __forceinline__ bool task_qkv(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  constexpr int NR = CPL == 1 ? 8 : (CPL == 2 ? 4 : (CPL == 3 ? 3 : 2));
  const int l = t.layer, g = t.a0, p0 = t.a1, np = t.a2, nj = 2 * np;
  const int H = a.H, D = a.D;
  const int QR = (a.Hq + 2 * a.Hkv) * D;
  const int TC = task_tc(t);
  const uint16_t* W = a.wqkv + (size_t)l * QR * H;
  auto rowptr = [&](int j) {
    int head, i, row;
    qkv_pair(p0 + (j >> 1), g, a.HG, D, a.Hq, a.Hkv, &head, &i, &row);
    row += (j & 1) * (D / 2);
    return (const uint4*)(W + (size_t)row * H);
  };
  float u[CPL * 8];
  auto ready = [&]() -> bool {
    if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
    const float* xf;
    const uint16_t* xb;
    layer_input(a, l, &xf, &xb);
    load_slice<CPL>(a, xf, xb, a.attn_norm + (size_t)l * H, H, TC, u, s.aux);
    return true;
  };
  if (!gemv_block<CPL, NR>(nj, TC, rowptr, ready, s.main, u)) return false;
  const int pos = a.seq_lens[0];
  const bool in_bounds = pos >= 0 && pos + 1 <= a.bound && pos < a.n_rope;
  int32_t phys = -1;
  if (in_bounds) phys = a.page_table[pos >> 4];
  const bool page_ok = in_bounds && phys >= 0 && phys < a.n_pages;
  if (!page_ok && threadIdx.x == 0) raise_status(a, DS_BOUNDS, ti, (uint32_t)pos, (uint32_t)phys);
  for (int q = threadIdx.x; q < np; q += NT) {
    const float y0 = job_sum(s.main, nj, TC, 2 * q), y1 = job_sum(s.main, nj, TC, 2 * q + 1);
    int head, i, row;
    const int sec = qkv_pair(p0 + q, g, a.HG, D, a.Hq, a.Hkv, &head, &i, &row);
    if (!page_ok) continue;
    float r0 = y0, r1 = y1;
    if (sec < 2) {
      const float c = a.rope_cos[(size_t)pos * (D / 2) + i];
      const float sn = a.rope_sin[(size_t)pos * (D / 2) + i];
      r0 = y0 * c - y1 * sn;
      r1 = y1 * c + y0 * sn;
    }
    if (sec == 0) {
      float* qd = a.q + (size_t)l * a.s_q + (size_t)head * D;
      qd[i] = r0;
      qd[i + D / 2] = r1;
    } else {
      uint16_t* base = a.pool + (size_t)phys * a.page_stride + (size_t)l * a.layer_stride +
                       (size_t)g * 2 * 16 * D;
      const int slot = pos & 15;
      if (sec == 1) {
        base[slot * D + i] = (uint16_t)f2bf(r0);
        base[slot * D + i + D / 2] = (uint16_t)f2bf(r1);
      } else {
        base[16 * D + i * 16 + slot] = (uint16_t)f2bf(r0);
        base[16 * D + (i + D / 2) * 16 + slot] = (uint16_t)f2bf(r1);
      }
    }
  }
  return true;
}

template <int D>
__device__ __forceinline__ bool task_attn(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  constexpr int KQ = D / 4;     // dims of one lane group in the QK product
  constexpr int NK4 = D / 32;   // 16-byte K loads per lane per page
  constexpr int NB = D / 16;    // 16-dim blocks of the PV product
  constexpr int NS = D / 16;    // MFMA k-steps of the QK product
  const int l = t.layer, b = t.a0, g = t.a1, pg0 = t.a2, npg = t.a3, split = t.aux;
  const int HG = a.HG;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int pos = a.seq_lens[b];
  const int n_tok = min(pos + 1, a.bound);
  const int pg_lim = min(pg0 + npg, (n_tok + 15) >> 4);
  const int first = pg0 + w;
  const int cnt = first < pg_lim ? (pg_lim - first + NWAVE - 1) / NWAVE : 0;
  const int cur = pos >> 4;
  const uint16_t* lbase = a.pool + (size_t)l * a.layer_stride + (size_t)g * 2 * 16 * D;
  const int32_t* prow = a.page_table + (size_t)b * a.max_pages;
  uint4 k0[NK4], k1[NK4];
  uint2 v0[NB], v1[NB];
  bool bad = false;
  auto load = [&](uint4 (&kk)[NK4], uint2 (&vv)[NB], int pg) {
    const int32_t phys = prow[pg];
    if (phys < 0 || phys >= a.n_pages) {
      bad = true;
#pragma unroll
      for (int i = 0; i < NK4; ++i) kk[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NB; ++i) vv[i] = make_uint2(0, 0);
      return;
    }
    const uint16_t* base = lbase + (size_t)phys * a.page_stride;
    const uint4* kp = (const uint4*)(base + r16 * D + kq * KQ);
#pragma unroll
    for (int i = 0; i < NK4; ++i) kk[i] = ld_nt(kp + i);
    const uint16_t* vp = base + 16 * D + r16 * 16 + kq * 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vv[nb] = ld_nt2((const uint2*)(vp + nb * 256));
  };
  const int pA = first, pB = first + NWAVE;
  const bool preA = cnt > 0 && pA < cur;
  const bool preB = cnt > 1 && pB < cur;
  if (preA) load(k0, v0, pA);
  if (preB) load(k1, v1, pB);
  if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
  if (cnt > 0 && !preA) load(k0, v0, pA);
  if (cnt > 1 && !preB) load(k1, v1, pB);

  // query operand: column r16 < 8 carries bf16(q) of head r16, column
  // r16 >= 8 the bf16 residual q - bf16(q) of head r16 - 8
  const int hh = r16 & 7;
  const bool lo_part = r16 >= 8;
  v4s qop[NS];
  {
    const bool valid = hh < HG;
    const float* qp = a.q + (size_t)l * a.s_q + (size_t)(g * HG + (valid ? hh : 0)) * D + kq * KQ;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const float4 x = valid ? *(const float4*)(qp + 4 * st) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hi = f2bf(xs[j]);
        const uint32_t v = lo_part ? f2bf(xs[j] - bf2f((uint16_t)hi)) : hi;
        qop[st][j] = (short)v;
      }
    }
  }
  float m_run = NEG_INF, l_run = 0.f;
  v4f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  const float scale = a.attn_scale;
  auto compute = [&](const uint4 (&kk)[NK4], const uint2 (&vv)[NB], int pg) {
    v4f S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const uint4 kv = kk[st >> 1];
      typedef unsigned u2v __attribute__((ext_vector_type(2)));
      const u2v pr = (st & 1) ? u2v{kv.z, kv.w} : u2v{kv.x, kv.y};
      S = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, pr), qop[st], S, 0, 0, 0);
    }
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = (S[j] + __shfl_xor(S[j], 8, 64)) * scale;
      sv[j] = (pg * 16 + 4 * kq + j) < n_tok ? x : NEG_INF;
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m_run, mx);
    const float alpha = mn == NEG_INF ? 1.f : expf(m_run - mn);
    float pj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pj[j] = sv[j] == NEG_INF ? 0.f : expf(sv[j] - mn);
    float ps = (pj[0] + pj[1]) + (pj[2] + pj[3]);
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = mn;
    v4s P;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hi = f2bf(pj[j]);
      P[j] = (short)(lo_part ? f2bf(pj[j] - bf2f((uint16_t)hi)) : hi);
    }
    float aj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) aj[j] = __shfl(alpha, (4 * kq + j) & 7, 64);
    // Slots at or past the live context may hold stale bits (even NaN) from an
    // earlier owner of the page: their probability is 0, but 0 * NaN is not,
    // so this lane's four V slots 4kq .. 4kq+3 are zeroed where invalid.
    const int valid = n_tok - pg * 16;
    uint32_t mlo = 0xFFFFFFFFu, mhi = 0xFFFFFFFFu;
    if (valid < 16) {
      const int s0 = 4 * kq;
      mlo = (s0 < valid ? 0x0000FFFFu : 0u) | (s0 + 1 < valid ? 0xFFFF0000u : 0u);
      mhi = (s0 + 2 < valid ? 0x0000FFFFu : 0u) | (s0 + 3 < valid ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[nb][j] *= aj[j];
      const uint2 vm = make_uint2(vv[nb].x & mlo, vv[nb].y & mhi);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(P, __builtin_bit_cast(v4s, vm), acc[nb], 0, 0, 0);
    }
  };
  for (int i = 0; i < cnt; i += 2) {
    compute(k0, v0, first + i * NWAVE);
    if (i + 2 < cnt) load(k0, v0, first + (i + 2) * NWAVE);
    if (i + 1 < cnt) {
      compute(k1, v1, first + (i + 1) * NWAVE);
      if (i + 3 < cnt) load(k1, v1, first + (i + 3) * NWAVE);
    }
  }
  if (bad && lane == 0) raise_status(a, DS_BOUNDS, ti, (uint32_t)b, 0xFFFFFFFFu);
  // merge hi/lo rows and publish this wave's partial in LDS
  float* Ow = s.main;                     // [NWAVE][HG][D]
  float* mw = s.aux;                      // [NWAVE][8]
  float* lw = s.aux + NWAVE * 8;          // [NWAVE][8]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float o = acc[nb][j] + __shfl_xor(acc[nb][j], 32, 64);
      const int head = 4 * kq + j;
      if (kq < 2 && head < HG) Ow[(w * HG + head) * D + nb * 16 + r16] = o;
    }
  if (lane < 8) {
    mw[w * 8 + lane] = m_run;
    lw[w * 8 + lane] = l_run;
  }
  __syncthreads();
  const int PS = D + 4;
  for (int idx = threadIdx.x; idx < HG * D; idx += NT) {
    const int head = idx / D, dim = idx % D;
    float M = NEG_INF;
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) M = fmaxf(M, mw[q * 8 + head]);
    float oo = 0.f, LL = 0.f;
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) {
      const float m = mw[q * 8 + head];
      const float e = m == NEG_INF ? 0.f : expf(m - M);
      oo += e * Ow[(q * HG + head) * D + dim];
      LL += e * lw[q * 8 + head];
    }
    float* dst = a.part + (size_t)l * a.s_part +
                 ((size_t)(b * a.Hq + g * HG + head) * a.S_max + split) * PS;
    dst[dim] = oo;
    if (dim == 0) {
      dst[D] = M;
      dst[D + 1] = LL;
    }
  }
  return true;
}

__device__ __forceinline__ bool task_comb(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  const int l = t.layer, b = t.a0, h = t.a1, S = t.a3, D = a.D, PS = D + 4;
  if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
  const float* base = a.part + (size_t)l * a.s_part + (size_t)(b * a.Hq + h) * a.S_max * PS;
  float* ms = s.aux;          // [S]
  float* ls = s.aux + 1024;   // [S]
  float* cs = s.aux + 2048;   // [S]
  for (int q = threadIdx.x; q < S; q += NT) {
    ms[q] = base[(size_t)q * PS + D];
    ls[q] = base[(size_t)q * PS + D + 1];
  }
  __syncthreads();
  float M = NEG_INF;
  for (int q = 0; q < S; ++q) M = fmaxf(M, ms[q]);
  float L = 0.f;
  for (int q = 0; q < S; ++q) L += ms[q] == NEG_INF ? 0.f : expf(ms[q] - M) * ls[q];
  for (int q = threadIdx.x; q < S; q += NT)
    cs[q] = (ms[q] == NEG_INF || L == 0.f) ? 0.f : expf(ms[q] - M) / L;
  __syncthreads();
  const int G = NT / D, sg = threadIdx.x / D, dim = threadIdx.x % D;
  float acc = 0.f;
  for (int q = sg; q < S; q += G) acc += cs[q] * base[(size_t)q * PS + dim];
  s.main[sg * D + dim] = acc;
  __syncthreads();
  if (threadIdx.x < D) {
    float o = 0.f;
    for (int q = 0; q < G; ++q) o += s.main[q * D + threadIdx.x];
    a.o[(size_t)l * a.s_o + (size_t)b * a.Hq * D + (size_t)h * D + threadIdx.x] = o;
  }
  return true;
}

template <int CPL>
__device__ __forceinline__ bool task_o(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  constexpr int NR = CPL == 1 ? 8 : (CPL == 2 ? 4 : (CPL == 3 ? 3 : 2));
  const int l = t.layer, r0 = t.a1, n = t.a2;
  const int H = a.H, K = a.Hq * a.D;
  const int TC = task_tc(t);
  const uint16_t* W = a.wo + (size_t)l * H * K;
  auto rowptr = [&](int j) { return (const uint4*)(W + (size_t)(r0 + j) * K); };
  float u[CPL * 8];
  auto ready = [&]() -> bool {
    if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
    load_slice<CPL>(a, a.o + (size_t)l * a.s_o, nullptr, nullptr, K, TC, u, s.aux);
    return true;
  };
  if (!gemv_block<CPL, NR>(n, TC, rowptr, ready, s.main, u)) return false;
  const float* xf;
  const uint16_t* xb;
  layer_input(a, l, &xf, &xb);
  for (int j = threadIdx.x; j < n; j += NT) {
    const float x = xf ? xf[r0 + j] : bf2f(xb[r0 + j]);
    a.xa[(size_t)l * a.s_x + r0 + j] = x + job_sum(s.main, n, TC, j);
  }
  return true;
}

template <int CPL>
__device__ __forceinline__ bool task_router(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  constexpr int NR = CPL == 1 ? 8 : (CPL == 2 ? 4 : (CPL == 3 ? 3 : 2));
  const int l = t.layer, r0 = t.a1, n = t.a2, H = a.H;
  const int TC = task_tc(t);
  const uint16_t* W = a.router + (size_t)l * a.E * H;
  auto rowptr = [&](int j) { return (const uint4*)(W + (size_t)(r0 + j) * H); };
  float u[CPL * 8];
  auto ready = [&]() -> bool {
    if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
    load_slice<CPL>(a, a.xa + (size_t)l * a.s_x, nullptr, a.ffn_norm + (size_t)l * H, H, TC, u, s.aux);
    return true;
  };
  if (!gemv_block<CPL, NR>(n, TC, rowptr, ready, s.main, u)) return false;
  for (int j = threadIdx.x; j < n; j += NT)
    a.rlog[(size_t)l * a.s_rlog + r0 + j] = job_sum(s.main, n, TC, j);
  return true;
}

template <int CPL>
__device__ __forceinline__ bool task_gateup(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  constexpr int NR = CPL == 1 ? 8 : (CPL == 2 ? 4 : (CPL == 3 ? 3 : 2));
  const int l = t.layer, slot = t.aux, f0 = t.a1, n = t.a2, nj = 2 * n;
  const int H = a.H, F = a.F, EE = a.dense ? 1 : a.E;
  const int TC = task_tc(t);
  int e = 0;
  if (!a.dense) {
    if (!wg_wait(a, t.wait_a, t.cnt_a, ti, &s.flag, s.tw)) return false;
    route(a, l, s);
    e = s.route_ids[slot];
    if ((t.flags & TF_WRITE_TOPK) && threadIdx.x < a.K) {
      if (a.topk_ids) a.topk_ids[(size_t)l * a.K + threadIdx.x] = s.route_ids[threadIdx.x];
      if (a.topk_w) a.topk_w[(size_t)l * a.K + threadIdx.x] = s.route_w[threadIdx.x];
    }
  }
  const uint16_t* Wg = a.gate + ((size_t)l * EE + e) * F * H;
  const uint16_t* Wu = a.up + ((size_t)l * EE + e) * F * H;
  auto rowptr = [&](int j) {
    return (const uint4*)(((j & 1) ? Wu : Wg) + (size_t)(f0 + (j >> 1)) * H);
  };
  float u[CPL * 8];
  auto ready = [&]() -> bool {
    if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
    load_slice<CPL>(a, a.xa + (size_t)l * a.s_x, nullptr, a.ffn_norm + (size_t)l * H, H, TC, u, s.aux);
    return true;
  };
  if (!gemv_block<CPL, NR>(nj, TC, rowptr, ready, s.main, u)) return false;
  float* act = a.act + (size_t)l * a.s_act + (size_t)slot * F;
  for (int q = threadIdx.x; q < n; q += NT) {
    const float yg = job_sum(s.main, nj, TC, 2 * q), yu = job_sum(s.main, nj, TC, 2 * q + 1);
    act[f0 + q] = yg / (1.0f + expf(-yg)) * yu;
  }
  return true;
}

template <int CPL>
__device__ __forceinline__ bool task_down(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  constexpr int NR = CPL == 1 ? 8 : (CPL == 2 ? 4 : (CPL == 3 ? 3 : 2));
  const int l = t.layer, r0 = t.a1, n = t.a2;
  const int H = a.H, F = a.F, KK = a.dense ? 1 : a.K, EE = a.dense ? 1 : a.E;
  const int nj = n * KK;
  const int TC = task_tc(t);
  if (!a.dense) {
    if (!wg_wait(a, t.wait_a, t.cnt_a, ti, &s.flag, s.tw)) return false;
    route(a, l, s);
  } else if (threadIdx.x == 0) {
    s.route_ids[0] = 0;
    s.route_w[0] = 1.f;
  }
  if (a.dense) __syncthreads();
  const uint16_t* Wd = a.down + (size_t)l * EE * H * F;
  auto rowptr = [&](int j) {
    const int e = s.route_ids[j % KK];
    return (const uint4*)(Wd + ((size_t)e * H + r0 + j / KK) * F);
  };
  const int my_slot = (threadIdx.x / TC) % KK;  // NT/TC is a multiple of KK
  float u[CPL * 8];
  auto ready = [&]() -> bool {
    if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
    load_slice<CPL>(a, a.act + (size_t)l * a.s_act + (size_t)my_slot * F, nullptr, nullptr, F, TC,
                    u, s.aux);
    return true;
  };
  if (!gemv_block<CPL, NR>(nj, TC, rowptr, ready, s.main, u)) return false;
  for (int q = threadIdx.x; q < n; q += NT) {
    float y = 0.f;
    for (int j = 0; j < KK; ++j) y += s.route_w[j] * job_sum(s.main, nj, TC, q * KK + j);
    a.xf[(size_t)l * a.s_x + r0 + q] = a.xa[(size_t)l * a.s_x + r0 + q] + y;
  }
  return true;
}

template <int CPL>
__device__ __forceinline__ bool task_lm(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  constexpr int NR = CPL == 1 ? 8 : (CPL == 2 ? 4 : (CPL == 3 ? 3 : 2));
  const int r0 = t.a1, n = t.a2, H = a.H;
  const int TC = task_tc(t);
  auto rowptr = [&](int j) { return (const uint4*)(a.lm + (size_t)(r0 + j) * H); };
  float u[CPL * 8];
  auto ready = [&]() -> bool {
    if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
    load_slice<CPL>(a, a.xf + (size_t)(a.L - 1) * a.s_x, nullptr, a.final_norm, H, TC, u, s.aux);
    return true;
  };
  if (!gemv_block<CPL, NR>(n, TC, rowptr, ready, s.main, u)) return false;
  float bv = NEG_INF;
  int bi = 0x7fffffff;
  for (int j = threadIdx.x; j < n; j += NT) {
    const float y = job_sum(s.main, n, TC, j);
    if (a.logits) a.logits[r0 + j] = y;
    if (y > bv) { bv = y; bi = r0 + j; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  float* rv = s.aux;
  int* ri = (int*)(s.aux + NWAVE);
  if ((threadIdx.x & 63) == 0) { rv[threadIdx.x >> 6] = bv; ri[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int q = 1; q < NWAVE; ++q)
      if (rv[q] > bv || (rv[q] == bv && ri[q] < bi)) { bv = rv[q]; bi = ri[q]; }
    // the wave-0 value of bv/bi is already folded in (lane 0 holds the wave result)
    a.lmpart[(size_t)t.a3 * 2] = __float_as_uint(bv);
    a.lmpart[(size_t)t.a3 * 2 + 1] = (uint32_t)bi;
  }
  return true;
}

__device__ __forceinline__ bool task_final(const KArgs& a, const Task& t, uint32_t ti, Smem& s) {
  if (!wg_wait(a, t.wait_b, t.cnt_b, ti, &s.flag, s.tw + 2)) return false;
  float bv = NEG_INF;
  int bi = 0x7fffffff;
  for (int q = threadIdx.x; q < t.a0; q += NT) {
    const float v = __uint_as_float(a.lmpart[(size_t)q * 2]);
    const int i = (int)a.lmpart[(size_t)q * 2 + 1];
    if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  float* rv = s.aux;
  int* ri = (int*)(s.aux + NWAVE);
  if ((threadIdx.x & 63) == 0) { rv[threadIdx.x >> 6] = bv; ri[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int q = 1; q < NWAVE; ++q)
      if (rv[q] > bv || (rv[q] == bv && ri[q] < bi)) { bv = rv[q]; bi = ri[q]; }
    a.tok_out[0] = bi;
    a.seq_lens[0] = a.seq_lens[0] + 1;
  }
  return true;
}

#define MK_CPL_DISPATCH(fn, K)                                  \
  [&]() -> bool {                                               \
    switch ((K) / (8 * task_tc(t))) {                           \
      case 1: return fn<1>(a, t, ti, s);                        \
      case 2: return fn<2>(a, t, ti, s);                        \
      case 3: return fn<3>(a, t, ti, s);                        \
      default: return fn<4>(a, t, ti, s);                       \
    }                                                           \
  }()

__global__ void __launch_bounds__(NT) megakernel(KArgs a) {
  __shared__ Smem s;
  const uint32_t* hdr = a.plan;
  const uint32_t* off = hdr + PLAN_HDR_WORDS;
  const Task* tasks = (const Task*)((const char*)a.plan + hdr[H_TASK_OFF_BYTES]);
  const uint32_t beg = off[blockIdx.x], end = off[blockIdx.x + 1];
  for (uint32_t ti = beg; ti < end; ++ti) {
    const Task t = tasks[ti];
    uint64_t t_start = 0;
    if (a.trace && threadIdx.x == 0) {
      t_start = __builtin_amdgcn_s_memrealtime();
      s.tw[0] = s.tw[1] = s.tw[2] = s.tw[3] = 0;
    }
    bool ok = true;
    switch (t.op) {
      case OP_QKV: ok = MK_CPL_DISPATCH(task_qkv, a.H); break;
      case OP_ATTN: ok = a.D == 128 ? task_attn<128>(a, t, ti, s) : task_attn<64>(a, t, ti, s); break;
      case OP_COMB: ok = task_comb(a, t, ti, s); break;
      case OP_O: ok = MK_CPL_DISPATCH(task_o, a.Hq * a.D); break;
      case OP_ROUTER: ok = MK_CPL_DISPATCH(task_router, a.H); break;
      case OP_GATEUP: ok = MK_CPL_DISPATCH(task_gateup, a.H); break;
      case OP_DOWN: ok = MK_CPL_DISPATCH(task_down, a.F); break;
      case OP_LM: ok = MK_CPL_DISPATCH(task_lm, a.H); break;
      case OP_FINAL: ok = task_final(a, t, ti, s); break;
      default: break;
    }
    if (!ok) return;
    uint64_t t_body = 0;
    if (a.trace && threadIdx.x == 0) t_body = __builtin_amdgcn_s_memrealtime();
    wg_signal(a, t.signal);
    if (a.trace && threadIdx.x == 0) {
      uint64_t* tr = a.trace + (size_t)ti * TRACE_WORDS;
      tr[0] = t_start;
      tr[1] = s.tw[0]; tr[2] = s.tw[1]; tr[3] = s.tw[2]; tr[4] = s.tw[3];
      tr[5] = t_body;
      tr[6] = __builtin_amdgcn_s_memrealtime();
      tr[7] = ((uint64_t)blockIdx.x << 32) | ((uint64_t)t.op << 16) | t.layer;
    }
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
    case mk::DS_TIMEOUT:
      return fail(MK_ETIMEOUT, "device wait timed out: task " + std::to_string(h[1]) + " counter " +
                                   std::to_string(h[2]) + " value " + std::to_string(h[3]));
    case mk::DS_BOUNDS:
      return fail(MK_EBOUNDS, "device bounds check failed: task " + std::to_string(h[1]) +
                                  " (position or page outside the plan/pool)");
    default:
      return fail(MK_EDEVICE, "unknown device status " + std::to_string(h[0]));
  }
}

extern "C" mk_status mk_decode_step(const mk_plan_t* p, const mk_weights* w, const mk_kv* kv,
                                    const mk_io* io, const mk_step_buffers* bu, uint32_t epoch,
                                    uint32_t timeout_ms, void* stream) {
  if (!p || !w || !kv || !io || !bu) return fail(MK_EINVAL, "mk_decode_step: NULL argument");
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
  if (!bu->plan || bu->plan_bytes < p->image.size() || !bu->workspace ||
      bu->workspace_bytes < p->ws_total || !bu->counters ||
      bu->counter_bytes < p->targets.size() * mk::CTR_STRIDE * 4 || !bu->status)
    return fail(MK_EINVAL, "mk_decode_step: step buffers missing or too small");
  if (epoch == 0 || (uint64_t)epoch * 65535ull >= (1ull << 32))
    return fail(MK_EBOUNDS, "mk_decode_step: epoch outside [1, 65536)");

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
  a.pool = (uint16_t*)kv->pool;
  a.layer_stride = (int64_t)m.n_kv_heads * 2 * 16 * m.head_dim;
  a.page_stride = (int64_t)m.n_layers * a.layer_stride;
  a.n_pages = kv->n_pages; a.page_table = kv->page_table; a.seq_lens = kv->seq_lens;
  a.rope_cos = kv->rope_cos; a.rope_sin = kv->rope_sin; a.n_rope = kv->n_rope_pos; a.bound = p->bound;
  a.tok_in = io->tokens_in; a.tok_out = io->tokens_out; a.topk_ids = io->topk_ids;
  a.topk_w = io->topk_w; a.logits = io->logits;
  char* ws = (char*)bu->workspace;
  a.xa = (float*)(ws + p->ws_off[MK_BUF_XATTN]); a.xf = (float*)(ws + p->ws_off[MK_BUF_XFFN]);
  a.q = (float*)(ws + p->ws_off[MK_BUF_Q]); a.part = (float*)(ws + p->ws_off[MK_BUF_PART]);
  a.o = (float*)(ws + p->ws_off[MK_BUF_O]); a.rlog = (float*)(ws + p->ws_off[MK_BUF_RLOG]);
  a.act = (float*)(ws + p->ws_off[MK_BUF_ACT]); a.lmpart = (uint32_t*)(ws + p->ws_off[MK_BUF_LMPART]);
  a.s_x = (int64_t)(p->ws_stride[MK_BUF_XATTN] / 4); a.s_q = (int64_t)(p->ws_stride[MK_BUF_Q] / 4);
  a.s_part = (int64_t)(p->ws_stride[MK_BUF_PART] / 4); a.s_o = (int64_t)(p->ws_stride[MK_BUF_O] / 4);
  a.s_rlog = (int64_t)(p->ws_stride[MK_BUF_RLOG] / 4); a.s_act = (int64_t)(p->ws_stride[MK_BUF_ACT] / 4);
  a.S_max = p->S_max; a.n_lm = p->n_lm;
  a.plan = (const uint32_t*)bu->plan; a.ctr = bu->counters; a.status = bu->status; a.epoch = epoch;
  a.timeout_ticks = (uint64_t)(timeout_ms ? timeout_ms : 2000) * 100000ull;
  if (bu->trace) {
    if (bu->trace_bytes < p->n_tasks * mk::TRACE_WORDS * sizeof(uint64_t))
      return fail(MK_EINVAL, "mk_decode_step: trace buffer smaller than 64 bytes per task");
    a.trace = bu->trace;
  }

  void* args[] = {&a};
  hipError_t e = hipLaunchCooperativeKernel((const void*)mk::dev::megakernel, dim3(p->n_cu),
                                            dim3(mk::NT), args, 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipLaunchCooperativeKernel(megakernel)");
  return MK_OK;
}
