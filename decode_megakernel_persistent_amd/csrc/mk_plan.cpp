// Host planner: decomposes one decode step into tile tasks, deals them over
// the compute units, allocates dependency counters, lays out the workspace,
// and checks the result (validate) or executes it on virtual compute units
// (simulate). Pure host code: no device is touched (kern page, "The runtime":
// state decisions made as pure host code are tested without a GPU).
//
// The decomposition follows the megakernel page ("What is a Megakernel?" and
// the caption of Image 2): every operation of the step is cut into tiles, one
// task per tile; the host deals the tasks round-robin over the compute units
// so each unit gets its own list in device memory; every task names the
// producer classes it waits for and the completion counter it increments.
// Stages, in order, per layer:
//   QKV (per kv group: q, k, v rows of the group, rotary epilogue, KV append)
//   ATTN (per sequence, kv group and page range: split-KV partials)
//   COMB (per sequence, query head and dim range: log-sum-exp merge)
//   O    (rows of W_o, residual)
//   ROUTER (MoE: rows of W_router)
//   EXPERT (at most one per unit: a gate/up tile of one expert slot with
//           SwiGLU, then a down tile of hidden rows over every slot with the
//           weighted combine and residual; the down part reads the
//           activations of every expert task of the layer)
// then LM (rows of the LM head, local argmax) and FINAL (argmax merge).
#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <numeric>
#include <random>
#include <set>
#include <string>
#include <tuple>
#include <queue>
#include <vector>

#include "mk.h"
#include "mk_plan.hpp"

using mk::Task;
using mkh::fail;

extern "C" mk_status mk_device_cu_count(int32_t* n_cu);

namespace {

std::vector<std::pair<int, int>> split_even(int n, int t) {
  std::vector<std::pair<int, int>> r;
  if (n <= 0) return r;
  t = std::max(1, std::min(t, n));
  int base = n / t, extra = n % t, s = 0;
  for (int i = 0; i < t; ++i) {
    int c = base + (i < extra ? 1 : 0);
    r.push_back({s, c});
    s += c;
  }
  return r;
}

Task mk_task(uint8_t op, int layer) {
  Task t;
  std::memset(&t, 0, sizeof t);
  t.op = op;
  t.layer = (uint16_t)layer;
  t.wait_a = t.wait_b = t.signal = mk::NO_CTR;
  return t;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Most rows one GEMV tile over reduction width K can hold in registers.
int rows_max(int K) {
  int tc = 0, cpl = 0;
  if (!mk::gemv_map(K, &tc, &cpl)) return 0;
  int rpw = std::min(mk::GEMV_RPW_MAX, mk::GEMV_REG_CHUNKS / cpl);
  return mk::gemv_groups(tc) * rpw;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Ranges of n items in units of u over t tasks: every range but the last is
// a whole number of units.
std::vector<std::pair<int, int>> split_units(int n, int u, int t) {
  auto r = split_even(ceil_div(n, u), t);
  for (auto& [s0, c] : r) {
    const int e = std::min(n, (s0 + c) * u);
    s0 *= u;
    c = e - s0;
  }
  return r;
}

// Row blocks (16 rows) per task of the MFMA batch projections: a task
// gathers every sequence's input once, so tasks are a few row blocks each.
constexpr int QKV_BLOCKS = 4, O_BLOCKS = 4, LM_BLOCKS = mk::MT_MAX_BLOCKS;
static_assert(8 * QKV_BLOCKS == mk::BQKV_PAIRS && mk::QPART_STRIDE == 2 * 8 * QKV_BLOCKS + 2,
              "batch QKV row blocks as the kernel reads their partial sums");
// words the reducing O task gathers into LDS (partials and residual)
constexpr int O_RED_WORDS = 16384;
// Batch 1 with attention on units of its own: an attention unit's QKV task
// takes this share of the rotary pairs of another unit's.
constexpr double QKV_ATTN_UNIT_SHARE = 0.5;

// Stages of a batch plan (B > 1), per layer:
//   BQKV  (16-row blocks of one kv group's rotary pairs, all sequences: MFMA
//          tile over one reduction block of the hidden state; blocks 1 ..
//          publish partial sums, block 0 adds them, then the rotary epilogue
//          and the KV append per sequence)
//   ATTN  (per sequence, kv group and page range of that sequence's bound)
//   COMB  (per sequence, query head and dim range)
//   BO    (16-row blocks of W_o, all sequences: MFMA tile over one reduction
//          block of the attention output; block 0 adds the others' partial
//          sums and the residual)
//   ROUTER (MoE, per sequence and range of router rows)
//   TOPK  (MoE, one per sequence: reads the router logits, softmax, top-k)
//   BEXP  (one expert, part q: gate/up rows with SwiGLU, then down rows, for
//          the sequences routed to it; the down part reads the activations of
//          every part of the same expert)
//   BCOMB (per sequence and hidden-row range: weighted sum of its experts'
//          outputs in slot order, plus the residual)
// then BLM (16-row blocks of the LM head, all sequences: MFMA tile,
// per-sequence argmax) and BFINAL (one per sequence).
mk_status batch_stages(mk_plan_t* p, const std::vector<int>& pages_b,
                       std::vector<std::vector<Task>>& stages) {
  const auto& m = p->m;
  const int L = m.n_layers, H = m.hidden, Hq = m.n_q_heads, Hkv = m.n_kv_heads, D = m.head_dim;
  const int B = p->B, HG = p->HG, n_cu = p->n_cu, F = p->F;
  const bool moe = m.n_experts > 0;
  const int NE = moe ? m.n_experts : 1;
  auto ctr16 = [](int c) { return c < 0 ? mk::NO_CTR : (uint16_t)c; };
  int P = std::max(1, n_cu / NE);
  P = std::min(P, std::min(F / 8, H / 16));
  p->n_exp_parts = P;
  const bool share = moe && NE <= mk::MAX_SHARE_EXPERTS && !(p->opts.flags & MK_PLAN_NO_EXPERT_SHARE);
  p->expert_share = share;
  if (NE * P > n_cu) return fail(MK_EUNSUPPORTED, "mk_plan: more expert tasks than compute units");
  // an expert task holds EXP_GROUP inputs of width H or F and up to 1024 result rows in LDS
  // expert GEMMs stream the reduction in groups of 8 k-steps of 32
  if (H % 256 || F % 256)
    return fail(MK_EUNSUPPORTED, "mk_plan: batch plans need hidden and FFN widths that are multiples of 256");
  if (H > 2048 || F > 2048 || 2 * ceil_div(F, P) > 1024 || ceil_div(H, P) > 1024)
    return fail(MK_EUNSUPPORTED, "mk_plan: batch expert tiles exceed LDS (hidden and FFN <= 2048, "
                                 "rows per expert task <= 1024): use more compute units");
  for (int l = 0; l < L; ++l) {
    {  // BQKV: 8 QKV_BLOCKS rotary pairs per row block, split over q_kb blocks
       // of the reduction: blocks 1 .. q_kb-1 publish partial sums (and
       // their sums of squares), then block 0 adds them, normalises, rotates
       // and appends
      const int KB = p->q_kb;
      for (int pass = 0; pass < 2; ++pass) {
        if (pass == 0 && KB == 1) continue;
        std::vector<Task> st;
        for (int g = 0; g < Hkv; ++g)
          for (int s0 = 0; s0 < p->n_pairs_g; s0 += 8 * QKV_BLOCKS)
            for (int kb = pass == 0 ? 1 : 0; kb < (pass == 0 ? KB : 1); ++kb) {
              Task t = mk_task(mk::OP_BQKV, l);
              t.wait_b = l == 0 ? mk::NO_CTR : ctr16(p->c_bcomb[l - 1]);
              // blocks 1 .. publish partial sums only: no completion counter
              t.signal = pass == 0 ? mk::NO_CTR : ctr16(p->c_qkv[l * Hkv + g]);
              t.a0 = g; t.a1 = s0; t.a2 = std::min(8 * QKV_BLOCKS, p->n_pairs_g - s0);
              t.units = (uint16_t)(pass == 0 ? 0 : 2 * t.a2);
              t.a3 = kb | (KB << 8);
              st.push_back(t);
            }
        stages.push_back(st);
      }
    }
    {  // ATTN
      std::vector<Task> st;
      for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g) {
          int si = 0;
          for (auto [s0, c] : split_even(pages_b[b], p->n_split[b])) {
            Task t = mk_task(mk::OP_ATTN, l);
            t.wait_b = ctr16(p->c_qkv[l * Hkv + g]);
            t.signal = ctr16(p->c_attn[l * Hkv + g]);
            t.a0 = b; t.a1 = g; t.a2 = s0; t.a3 = c; t.aux = (uint16_t)si++;
            t.units = (uint16_t)c;
            st.push_back(t);
          }
        }
      // longest splits first: dealt round-robin (the units' page counts even
      // out), or pulled from the queue in this order by one queue task per unit
      std::stable_sort(st.begin(), st.end(), [](const Task& x, const Task& y) { return x.a3 > y.a3; });
      if (p->attn_queue) {
        if (l == 0) {
          p->split_table = st;
          for (auto& t : p->split_table) t.layer = 0, t.wait_b = t.signal = mk::NO_CTR, t.units = 0;
        }
        std::vector<Task> qs;
        for (int i = 0; i < n_cu; ++i) {
          Task t = mk_task(mk::OP_ATTN, l);
          t.flags = mk::TF_QUEUE;
          t.wait_b = ctr16(p->c_qkv[l * Hkv]);
          t.signal = ctr16(p->c_attn[l * Hkv]);
          t.a0 = p->c_queue[l]; t.a1 = 0; t.a2 = (int32_t)p->split_table.size(); t.a3 = n_cu;
          t.units = 0;  // each split pulled adds its pages
          qs.push_back(t);
        }
        stages.push_back(qs);
      } else {
        stages.push_back(st);
      }
    }
    {  // COMB: whole heads (nh of one kv group per task) while there are more
       // (sequence, head) pairs than units, else as many dim ranges as fit
      std::vector<Task> st;
      int nh = 1;
      while (p->comb_dim_tasks == 1 && B * Hq / nh > n_cu && HG % (2 * nh) == 0 && 2 * nh * D <= mk::NT &&
             (int64_t)p->S_max * 2 * nh * (D + 2) <= mk::COMB_BATCH_WORDS)
        nh *= 2;
      for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; h += nh)
          for (auto [d0, nd] : split_even(nh * D, nh > 1 ? 1 : p->comb_dim_tasks)) {
            Task t = mk_task(mk::OP_COMB, l);
            t.wait_b = ctr16(p->c_attn[l * Hkv + h / HG]);
            t.signal = ctr16(p->c_comb[l]);
            t.a0 = b; t.a1 = h; t.a2 = d0; t.a3 = nd; t.aux = (uint16_t)p->n_split[b];
            t.units = (uint16_t)nd;
            st.push_back(t);
          }
      stages.push_back(st);
    }
    {  // BO, split over o_kb blocks of the reduction: every block publishes
       // the partial sums of its tile, then each of o_kb slices of a row
       // block adds the blocks' partial sums of its rows and the residual
       // (the reduction spread over as many tasks as the tiles)
      const int KB = p->o_kb;
      if (KB == 1) {
        std::vector<Task> st;
        for (int s0 = 0; s0 < H; s0 += 16 * O_BLOCKS) {
          Task t = mk_task(mk::OP_BO, l);
          t.wait_b = ctr16(p->c_comb[l]);
          t.signal = ctr16(p->c_o[l]);
          t.a0 = 0; t.a1 = s0; t.a2 = std::min(16 * O_BLOCKS, H - s0); t.a3 = 1;
          t.units = (uint16_t)t.a2;
          st.push_back(t);
        }
        stages.push_back(st);
      } else {
        std::vector<Task> tiles, sums;
        for (int s0 = 0; s0 < H; s0 += 16 * O_BLOCKS) {
          const int n = std::min(16 * O_BLOCKS, H - s0);
          for (int kb = 0; kb < KB; ++kb) {
            Task t = mk_task(mk::OP_BO, l);
            t.wait_b = ctr16(p->c_comb[l]);
            t.a0 = kb; t.a1 = s0; t.a2 = n; t.a3 = KB;
            tiles.push_back(t);
          }
          for (auto [r0, c] : split_even(n, KB)) {
            Task t = mk_task(mk::OP_BO, l);
            t.flags = mk::TF_REDUCE;
            t.wait_b = ctr16(p->c_comb[l]);
            t.signal = ctr16(p->c_o[l]);
            t.a1 = s0 + r0; t.a2 = c; t.a3 = KB;
            t.units = (uint16_t)c;
            sums.push_back(t);
          }
        }
        stages.push_back(tiles);
        stages.push_back(sums);
      }
    }
    if (moe) {  // ROUTER rows (a few tasks per sequence), then TOPK per sequence
      const int nr = std::max(1, std::min(std::min(8, m.n_experts), n_cu / B));
      std::vector<Task> rt;
      for (int b = 0; b < B; ++b)
        for (auto [r0, n] : split_even(m.n_experts, nr)) {
          Task t = mk_task(mk::OP_ROUTER, l);
          t.wait_b = ctr16(p->c_o[l]);
          t.signal = ctr16(p->c_router[l]);
          t.a0 = b; t.a1 = r0; t.a2 = n;
          t.units = (uint16_t)n;
          rt.push_back(t);
        }
      stages.push_back(rt);
      std::vector<Task> tk;
      for (int b = 0; b < B; ++b) {
        Task t = mk_task(mk::OP_TOPK, l);
        t.flags = mk::TF_LOGITS;
        t.wait_b = ctr16(p->c_router[l]);
        t.signal = ctr16(p->c_topk[l]);
        t.a0 = b;
        t.units = 1;
        tk.push_back(t);
      }
      stages.push_back(tk);
    }
    {  // BEXP: fixed (expert, part) per task, or shares of the chosen experts' rows
      std::vector<Task> st;
      const auto fr = split_units(F, 8, P), hr = split_units(H, 16, P);
      const int T = NE * P;
      const int64_t W = (int64_t)NE * (F + H);  // outputs per layer: every expert's rows
      for (int e = 0; e < NE; ++e)
        for (int q = 0; q < P; ++q) {
          Task t = mk_task(mk::OP_BEXP, l);
          t.wait_a = moe ? ctr16(p->c_topk[l]) : mk::NO_CTR;
          t.wait_b = ctr16(p->c_o[l]);
          t.signal = ctr16(p->c_expert[l]);
          if (share) {
            // the device assigns the rows; the counter counts every expert's
            // rows once per layer, an equal part per task
            const int i = e * P + q;
            t.flags |= mk::TF_SHARE;
            t.aux = (uint16_t)i;
            t.a1 = T;
            t.units = (uint16_t)(W * (i + 1) / T - W * i / T);
          } else {
            t.a0 = e;
            t.a1 = q < (int)fr.size() ? fr[q].first : 0;
            t.a2 = q < (int)fr.size() ? fr[q].second : 0;
            t.a3 = q < (int)hr.size() ? (hr[q].first << 16) | hr[q].second : 0;
            t.units = (uint16_t)(t.a2 + (t.a3 & 0xFFFF));
          }
          st.push_back(t);
        }
      stages.push_back(st);
    }
    {  // BCOMB: its words (slots x rows + residual rows + weights) fit the gather vector
      std::vector<Task> st;
      const int KK = moe ? m.top_k : 1;
      const int max_rows = std::max(16, (mk::dev_lds_vec() - KK) / (KK + 1) / 16 * 16);
      const int per_b = std::max(std::max(1, n_cu / B), ceil_div(H, max_rows));
      for (int b = 0; b < B; ++b)
        for (auto [s0, c] : split_units(H, 16, per_b)) {
          Task t = mk_task(mk::OP_BCOMB, l);
          t.wait_a = moe ? ctr16(p->c_topk[l]) : mk::NO_CTR;
          t.wait_b = ctr16(p->c_expert[l]);
          t.signal = ctr16(p->c_bcomb[l]);
          t.a0 = b; t.a1 = s0; t.a2 = c;
          t.units = (uint16_t)c;
          st.push_back(t);
        }
      stages.push_back(st);
    }
  }
  {  // BLM, BFINAL
    std::vector<Task> st;
    const int rows = 16 * LM_BLOCKS;
    int i = 0;
    for (int s0 = 0; s0 < m.vocab; s0 += rows) {
      Task t = mk_task(mk::OP_BLM, 0);
      t.wait_b = ctr16(p->c_bcomb[L - 1]);
      t.signal = ctr16(p->c_lm);
      t.a1 = s0; t.a2 = std::min(rows, m.vocab - s0); t.a3 = i++;
      t.units = (uint16_t)t.a2;
      st.push_back(t);
    }
    p->n_lm = i;
    if (p->n_lm > 4096) return fail(MK_EUNSUPPORTED, "mk_plan: more than 4096 LM-head tiles");
    stages.push_back(st);
    std::vector<Task> fin;
    for (int b = 0; b < B; ++b) {
      Task f = mk_task(mk::OP_BFINAL, 0);
      f.wait_b = ctr16(p->c_lm);
      f.a0 = p->n_lm; f.a1 = b;
      f.a2 = rows;  // rows per LM-head tile (the last may hold fewer)
      fin.push_back(f);
    }
    stages.push_back(fin);
  }
  return MK_OK;
}

}  // namespace

extern "C" mk_status mk_plan(const mk_model_desc* m, const mk_batch_desc* bd,
                             const mk_plan_opts* o, mk_plan_t** out) {
  if (!m || !bd || !out) return fail(MK_EINVAL, "mk_plan: NULL argument");
  *out = nullptr;
  const int L = m->n_layers, H = m->hidden, Hq = m->n_q_heads, Hkv = m->n_kv_heads,
            D = m->head_dim;
  const bool moe = m->n_experts > 0;
  if (L <= 0 || H <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || m->vocab <= 0)
    return fail(MK_EINVAL, "mk_plan: non-positive model dimension");
  if (Hq % Hkv) return fail(MK_EINVAL, "mk_plan: n_q_heads must be a multiple of n_kv_heads");
  if (m->page_tokens != 16) return fail(MK_EUNSUPPORTED, "mk_plan: page_tokens must be 16");
  if (D != 64 && D != 128) return fail(MK_EUNSUPPORTED, "mk_plan: head_dim must be 64 or 128");
  if (Hq / Hkv > 8) return fail(MK_EUNSUPPORTED, "mk_plan: more than 8 query heads per kv head");
  const int F = moe ? m->expert_ffn : m->ffn_dim;
  if (F <= 0) return fail(MK_EINVAL, "mk_plan: ffn width must be positive");
  if (moe && (m->top_k <= 0 || m->top_k > m->n_experts || m->top_k > 16 || m->n_experts > 256))
    return fail(MK_EUNSUPPORTED, "mk_plan: MoE needs 0 < top_k <= min(16, n_experts), n_experts <= 256");
  // activations pass between tasks as pairs of neighbouring tagged words
  // read together: every gathered run (hidden, heads x dim, top_k x FFN,
  // router logits) has an even length and starts at an even word
  if (moe && m->n_experts % 2)
    return fail(MK_EUNSUPPORTED, "mk_plan: the number of experts must be even");
  int tc, cpl;
  for (int K : {H, Hq * D, F})
    if (!mk::gemv_map(K, &tc, &cpl))
      return fail(MK_EUNSUPPORTED, "mk_plan: reduction width " + std::to_string(K) +
                                       " has no GEMV mapping (need K/8 a multiple of 32 with "
                                       "K/8/lanes in {1,2,3,4,6,8})");
  {
    int tcf = 64, cplf = 1;
    mk::gemv_map(F, &tcf, &cplf);
    int kk = moe ? m->top_k : 1;
    if (mk::gemv_groups(tcf) % kk)
      return fail(MK_EUNSUPPORTED, "mk_plan: down-projection lane groups (" +
                                       std::to_string(mk::gemv_groups(tcf)) + ") not a multiple of top_k");
    if (rows_max(F) < kk)
      return fail(MK_EUNSUPPORTED, "mk_plan: down-projection tile cannot hold top_k rows");
  }
  if ((size_t)H > 8192 || (size_t)Hq * D > 8192 || (size_t)(moe ? m->top_k : 1) * F > 8192)
    return fail(MK_EUNSUPPORTED, "mk_plan: an input vector exceeds the 8192-float LDS staging area");
  int kclass = -1;
  {
    kclass = mk::kernel_class(H, Hq * D, F, D);
    if (kclass < 0)
      return fail(MK_EUNSUPPORTED, "mk_plan: no compiled kernel variant for hidden " + std::to_string(H) +
                                       ", heads x dim " + std::to_string(Hq * D) + ", FFN " +
                                       std::to_string(F) + ", head dim " + std::to_string(D));
  }
  const int B = bd->batch;
  if (B < 1 || B > mk::MAX_BATCH)
    return fail(MK_EUNSUPPORTED, "mk_plan: batch must be 1 .. " + std::to_string(mk::MAX_BATCH));
  const bool batch = B > 1;
  if (batch) {
    for (int K : {H, Hq * D, F})
      if (K % mk::MT_KP)
        return fail(MK_EUNSUPPORTED, "mk_plan: batch plans need hidden, heads x dim and FFN widths "
                                     "that are multiples of " + std::to_string(mk::MT_KP));
    if (moe && B * m->top_k > mk::NT)
      return fail(MK_EUNSUPPORTED, "mk_plan: batch x top_k must be at most " + std::to_string(mk::NT));
  }
  if (m->page_tokens != 16) return fail(MK_EUNSUPPORTED, "mk_plan: page_tokens must be 16");
  if (!bd->seq_lens || !bd->page_table || bd->max_pages <= 0)
    return fail(MK_EINVAL, "mk_plan: seq_lens / page_table / max_pages missing");
  const int max_bound = bd->max_ctx_bound;
  if (max_bound <= 0 || (max_bound + 15) / 16 > bd->max_pages)
    return fail(MK_EBOUNDS, "mk_plan: max_ctx_bound needs " + std::to_string((max_bound + 15) / 16) +
                                " pages per sequence, page table has " + std::to_string(bd->max_pages));
  std::vector<int32_t> seq_bound(B);
  for (int b = 0; b < B; ++b) {
    const int bb = bd->ctx_bounds ? bd->ctx_bounds[b] : max_bound;
    if (bb <= 0 || bb > max_bound)
      return fail(MK_EBOUNDS, "mk_plan: ctx_bounds[" + std::to_string(b) + "] outside (0, max_ctx_bound]");
    seq_bound[b] = bb;
    if (bd->seq_lens[b] < 0 || bd->seq_lens[b] + 1 > bb)
      return fail(MK_EBOUNDS, "mk_plan: seq_lens[" + std::to_string(b) + "] + 1 exceeds its context bound");
    for (int j = 0; j < (bb + 15) / 16; ++j)
      if (bd->page_table[(int64_t)b * bd->max_pages + j] < 0)
        return fail(MK_EBOUNDS, "mk_plan: sequence " + std::to_string(b) +
                                    " has no page mapped at logical page " + std::to_string(j));
  }
  const bool prefill = o && (o->flags & MK_PLAN_PREFILL);
  if (prefill) {
    if (!batch) return fail(MK_EINVAL, "mk_plan: a prefill chunk has 2 .. 32 rows");
    for (int b = 1; b < B; ++b) {
      if (bd->seq_lens[b] != bd->seq_lens[0] + b)
        return fail(MK_EINVAL, "mk_plan: prefill rows must be consecutive positions of one sequence");
      for (int j = 0; j < bd->max_pages; ++j)
        if (bd->page_table[(int64_t)b * bd->max_pages + j] != bd->page_table[j])
          return fail(MK_EINVAL, "mk_plan: prefill rows must share one page-table row");
    }
  }
  // batch 1 runs with its own bound; a batch keeps max_ctx_bound as the plan bound
  const int bound = batch ? max_bound : seq_bound[0];
  const int pg_bound = (bound + 15) / 16;
  int n_cu = o && o->n_cu > 0 ? o->n_cu : 0;
  if (n_cu == 0) {
    if (mk_device_cu_count(&n_cu) != MK_OK || n_cu <= 0)
      return fail(MK_EINVAL, "mk_plan: opts.n_cu is 0 and no device could be queried");
  }
  if (n_cu > 4096) return fail(MK_EINVAL, "mk_plan: n_cu too large");

  auto* p = new mk_plan_t();
  static std::atomic<uint64_t> next_uid{1};
  p->uid = next_uid.fetch_add(1);
  p->m = *m;
  p->opts.n_cu = n_cu;
  p->opts.attn_split_pages = o ? o->attn_split_pages : 0;
  p->opts.flags = o ? o->flags : 0;
  p->B = B;
  p->max_pages = bd->max_pages;
  p->bound = bound;
  p->n_cu = n_cu;
  p->batch = batch;
  p->seq_bound = seq_bound;
  p->seq_lens.assign(bd->seq_lens, bd->seq_lens + B);
  p->page_table.assign(bd->page_table, bd->page_table + (int64_t)B * bd->max_pages);
  p->kernel_class = kclass;
  p->HG = Hq / Hkv;
  p->QKV_ROWS = (Hq + 2 * Hkv) * D;
  p->F = F;
  p->n_pairs_g = (p->HG * D + 2 * D) / 2;
  if (batch) {
    // O projection: row blocks of 16 O_BLOCKS rows, split over o_kb blocks of
    // the reduction (whole MT_KP panels) while about one task per unit
    // remains and the reducing task's words fit its LDS gather area
    const int Kq = Hq * D, n_rb = ceil_div(H, 16 * O_BLOCKS), npan = Kq / mk::MT_KP;
    int kb = 1;
    while (npan % (2 * kb) == 0 && n_rb * 2 * kb <= n_cu && 2 * kb * B * 16 * O_BLOCKS <= O_RED_WORDS)
      kb *= 2;
    p->o_kb = kb;
    // QKV projection: the same over the hidden state, while the reducing
    // task's words (partial rows and sums of squares) fit its gather area
    const int RS = 2 * 8 * QKV_BLOCKS + 2, npq = H / mk::MT_KP;
    p->q_rb = Hkv * ceil_div(p->n_pairs_g, 8 * QKV_BLOCKS);
    int qk = 1;
    while (npq % (2 * qk) == 0 && p->q_rb * 2 * qk <= n_cu && (2 * qk - 1) * B * RS <= O_RED_WORDS) qk *= 2;
    p->q_kb = qk;
  }
  const int HG = p->HG, K = moe ? m->top_k : 1;

  auto new_ctr = [&](const std::string& name) {
    p->targets.push_back(0);
    p->ctr_name.push_back(name);
    return (int32_t)p->targets.size() - 1;
  };
  // attention: static splits of about pg_total / n_cu pages each, or (when
  // asked for) a shared queue of QUEUE_PAGES-page splits that every compute
  // unit pulls from, so that units streaming faster take more of them. On
  // MI355X the static splits are faster even at 262144 tokens: a pulled split
  // restarts its page pipeline, its query gather and its merge.
  std::vector<int> pages_b(B);
  int pg_total = 0;
  for (int b = 0; b < B; ++b) {
    pages_b[b] = batch ? (seq_bound[b] + 15) / 16 : pg_bound;
    pg_total += pages_b[b] * Hkv;
  }
  const int flags = o ? o->flags : 0;
  int pps = o && o->attn_split_pages > 0 ? o->attn_split_pages : (pg_total + n_cu - 1) / n_cu;
  const bool queue = !(flags & MK_PLAN_NO_ATTN_QUEUE) && !prefill && (flags & MK_PLAN_ATTN_QUEUE);
  p->router_fold = !batch && moe && !(flags & MK_PLAN_NO_ROUTER_FOLD);
  if (queue && !batch) pps = mk::QUEUE_PAGES;
  // a batch: about four splits per unit, so that ragged lengths even out
  // (dealt statically, or pulled from the queue longest first)
  if (batch && !(o && o->attn_split_pages > 0)) pps = std::max(8, ceil_div(pg_total, 4 * n_cu));
  p->attn_queue = queue;
  // batch 1, static splits: when splits of two pages per wave fit on at most
  // 3/5 of the units, attention and its combine run on those units (set A)
  // and the O projection and router on the others (set B), so that the O
  // rows stream while attention runs
  int n_attn_units = 0;
  if (!batch && !queue && !(o && o->attn_split_pages > 0) && moe) {
    const int S = ceil_div(pg_bound, 2 * mk::NWAVE);
    if (Hkv * S <= (3 * n_cu) / 5 && Hkv * S >= n_cu / 4) {
      pps = ceil_div(pg_bound, S);
      n_attn_units = Hkv * S;
    }
  }
  for (int l = 0; l < L; ++l) {
    const std::string ls = std::to_string(l);
    if (batch) {
      for (int g = 0; g < Hkv; ++g) p->c_qkv.push_back(new_ctr("qkv[" + ls + "][" + std::to_string(g) + "]"));
      if (queue) {  // a queue task takes splits of any kv head: one attention counter per layer
        const int ca = new_ctr("attn[" + ls + "]");
        for (int g = 0; g < Hkv; ++g) p->c_attn.push_back(ca);
        p->c_queue.push_back(new_ctr("queue[" + ls + "]"));
      } else {
        for (int g = 0; g < Hkv; ++g) p->c_attn.push_back(new_ctr("attn[" + ls + "][" + std::to_string(g) + "]"));
      }
      p->c_comb.push_back(new_ctr("comb[" + ls + "]"));
      p->c_o.push_back(new_ctr("o[" + ls + "]"));
      p->c_router.push_back(moe ? new_ctr("router[" + ls + "]") : -1);
      p->c_topk.push_back(moe ? new_ctr("topk[" + ls + "]") : -1);
      p->c_expert.push_back(new_ctr("expert[" + ls + "]"));
      p->c_bcomb.push_back(new_ctr("ffn[" + ls + "]"));
      continue;
    }
    if (queue) {  // one QKV and one attention counter per layer: a queue task takes any group
      const int cq = new_ctr("qkv[" + ls + "]"), ca = new_ctr("attn[" + ls + "]");
      for (int g = 0; g < Hkv; ++g) p->c_qkv.push_back(cq), p->c_attn.push_back(ca);
      p->c_queue.push_back(new_ctr("queue[" + ls + "]"));
    } else {
      for (int g = 0; g < Hkv; ++g) p->c_qkv.push_back(new_ctr("qkv[" + ls + "][" + std::to_string(g) + "]"));
      for (int g = 0; g < Hkv; ++g) p->c_attn.push_back(new_ctr("attn[" + ls + "][" + std::to_string(g) + "]"));
    }
    p->c_comb.push_back(new_ctr("comb[" + ls + "]"));
    p->c_o.push_back(new_ctr("o[" + ls + "]"));
    p->c_router.push_back(moe ? new_ctr("router[" + ls + "]") : -1);
    p->c_expert.push_back(new_ctr("expert[" + ls + "]"));
  }
  p->c_lm = new_ctr("lm");
  if (p->targets.size() >= mk::NO_CTR) {
    delete p;
    return fail(MK_EUNSUPPORTED, "mk_plan: too many counters");
  }

  pps = std::max(std::max(1, pps), (pg_bound + 1023) / 1024);  // at most 1024 splits per (b, g)
  if (batch && pps > mk::NT) pps = mk::NT;
  if (pps > 2 * mk::NT) {
    delete p;
    return fail(MK_EUNSUPPORTED, "mk_plan: more than " + std::to_string(2 * mk::NT) + " pages per attention split");
  }
  p->n_split.assign(B, 0);
  for (int b = 0; b < B; ++b) p->n_split[b] = (pages_b[b] + pps - 1) / pps;
  if (batch && !(o && o->attn_split_pages > 0) && pg_total > 0) {
    // a batch: 4 n_cu splits in all, each sequence's share in proportion to
    // its pages (largest remainders), so that the splits are about equal and
    // come out at four per unit; at least one split per sequence, at least 8
    // and at most NT pages per split
    const int64_t T = std::max<int64_t>(B, 4LL * n_cu / std::max(1, Hkv));
    int64_t tot = 0;
    for (int b = 0; b < B; ++b) tot += pages_b[b];
    std::vector<std::pair<double, int>> rem;
    int64_t given = 0;
    for (int b = 0; b < B; ++b) {
      const double q = (double)pages_b[b] * (double)T / (double)std::max<int64_t>(1, tot);
      p->n_split[b] = std::max(1, (int)q);
      given += p->n_split[b];
      rem.push_back({q - std::floor(q), b});
    }
    std::stable_sort(rem.begin(), rem.end(), [](auto& x, auto& y) { return x.first > y.first; });
    for (size_t i = 0; i < rem.size() && given < T; ++i, ++given) p->n_split[rem[i].second]++;
    for (int b = 0; b < B; ++b) {
      const int lo = std::max(1, ceil_div(pages_b[b], mk::NT)), hi = std::max(1, ceil_div(pages_b[b], 8));
      p->n_split[b] = std::min(std::max(p->n_split[b], lo), std::max(lo, hi));
    }
  }
  p->S_max = *std::max_element(p->n_split.begin(), p->n_split.end());
  // combine tasks per (sequence, query head): a power of two (D is 64 or
  // 128, so every task takes an even run of dims), at most D / 8
  p->comb_dim_tasks = 1;
  const int comb_units = n_attn_units > 0 ? n_attn_units : n_cu;
  while (2 * p->comb_dim_tasks <= D / 8 && 2 * p->comb_dim_tasks * B * Hq <= comb_units) p->comb_dim_tasks *= 2;
  while (p->comb_dim_tasks < D / 8 && (size_t)p->S_max * (ceil_div(D, p->comb_dim_tasks) + 2) > 8192)
    p->comb_dim_tasks *= 2;  // fewer dims per combine task when there are many splits

  std::vector<std::vector<Task>> stages;
  auto ctr16 = [](int c) { return c < 0 ? mk::NO_CTR : (uint16_t)c; };
  if (batch) {
    mk_status st = batch_stages(p, pages_b, stages);
    if (st != MK_OK) {
      delete p;
      return st;
    }
  }
  for (int l = 0; l < L && !batch; ++l) {
    // QKV: tiles of rotary pairs within one kv group
    {
      std::vector<Task> st;
      int per_g = std::max(1, n_cu / Hkv);
      const int cap_pairs = std::max(1, rows_max(H) / 2);
      per_g = std::max(per_g, ceil_div(p->n_pairs_g, cap_pairs));
      auto qkv_task = [&](int g, int s0, int c) {
        Task t = mk_task(mk::OP_QKV, l);
        t.wait_b = l == 0 ? mk::NO_CTR : ctr16(p->c_expert[l - 1]);
        t.signal = ctr16(p->c_qkv[l * Hkv + g]);
        t.a0 = g; t.a1 = s0; t.a2 = c;
        t.units = (uint16_t)(2 * c);
        return t;
      };
      if (n_attn_units > 0 && per_g * Hkv == n_cu) {
        // unit i runs task i (group i mod Hkv); an attention unit takes
        // QKV_ATTN_UNIT_SHARE of the pairs of another unit, so that it starts
        // its split (and requests the pages not staged) earlier
        for (int i = 0; i < n_cu; ++i) st.push_back(Task{});
        for (int g = 0; g < Hkv; ++g) {
          std::vector<int> us;
          double wsum = 0.0;
          for (int i = g; i < n_cu; i += Hkv) {
            us.push_back(i);
            wsum += i < n_attn_units ? QKV_ATTN_UNIT_SHARE : 1.0;
          }
          std::vector<int> cnt(us.size());
          std::vector<std::pair<double, int>> rem;
          int given = 0;
          for (size_t k = 0; k < us.size(); ++k) {
            const double q = p->n_pairs_g * (us[k] < n_attn_units ? QKV_ATTN_UNIT_SHARE : 1.0) / wsum;
            cnt[k] = std::min(cap_pairs, (int)q);
            given += cnt[k];
            rem.push_back({q - std::floor(q), (int)k});
          }
          std::stable_sort(rem.begin(), rem.end(), [](auto& x, auto& y) { return x.first > y.first; });
          for (size_t k = 0; given < p->n_pairs_g; k = (k + 1) % rem.size())
            if (cnt[rem[k].second] < cap_pairs) cnt[rem[k].second]++, given++;
          int s0 = 0;
          for (size_t k = 0; k < us.size(); ++k) {
            st[us[k]] = qkv_task(g, s0, cnt[k]);
            s0 += cnt[k];
          }
        }
      } else {
        for (int g = 0; g < Hkv; ++g)
          for (auto [s0, c] : split_even(p->n_pairs_g, per_g)) st.push_back(qkv_task(g, s0, c));
      }
      stages.push_back(st);
    }
    // ATTN: split-KV tasks per (b, g), or one queue task per compute unit
    // pulling the splits of QUEUE_PAGES pages of every kv head (kv head major)
    if (queue) {
      if (l == 0) {
        p->split_table.clear();
        for (int g = 0; g < Hkv; ++g)
          for (int si = 0; si < p->n_split[0]; ++si) {
            Task t = mk_task(mk::OP_ATTN, 0);
            t.a0 = 0; t.a1 = g; t.a2 = si * mk::QUEUE_PAGES;
            t.a3 = std::min(mk::QUEUE_PAGES, pg_bound - t.a2); t.aux = (uint16_t)si;
            p->split_table.push_back(t);
          }
      }
      std::vector<Task> st;
      for (int i = 0; i < n_cu; ++i) {
        Task t = mk_task(mk::OP_ATTN, l);
        t.flags = mk::TF_QUEUE;
        t.wait_b = ctr16(p->c_qkv[l * Hkv]);
        t.signal = ctr16(p->c_attn[l * Hkv]);
        t.a0 = p->c_queue[l]; t.a1 = 0; t.a2 = (int32_t)p->split_table.size(); t.a3 = n_cu;
        t.units = 0;  // each split pulled adds its pages
        st.push_back(t);
      }
      stages.push_back(st);
    } else {
      std::vector<Task> st;
      for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g) {
          int si = 0;
          for (auto [s0, c] : split_even(pg_bound, p->n_split[b])) {
            Task t = mk_task(mk::OP_ATTN, l);
            t.wait_b = ctr16(p->c_qkv[l * Hkv + g]);
            t.signal = ctr16(p->c_attn[l * Hkv + g]);
            t.a0 = b; t.a1 = g; t.a2 = s0; t.a3 = c; t.aux = (uint16_t)si++;
            t.units = (uint16_t)c;
            st.push_back(t);
          }
        }
      // longest splits first: dealt round-robin, the units' page counts even out
      std::stable_sort(st.begin(), st.end(), [](const Task& x, const Task& y) { return x.a3 > y.a3; });
      stages.push_back(st);
    }
    // COMB: one query head of one sequence, a range of its dims, per task
    {
      std::vector<Task> st;
      for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h)
          for (auto [d0, nd] : split_even(D, p->comb_dim_tasks)) {
            Task t = mk_task(mk::OP_COMB, l);
            t.wait_b = ctr16(p->c_attn[l * Hkv + h / HG]);
            t.signal = ctr16(p->c_comb[l]);
            t.a0 = b; t.a1 = h; t.a2 = d0; t.a3 = nd; t.aux = (uint16_t)p->n_split[b];
            t.units = (uint16_t)nd;
            st.push_back(t);
          }
      stages.push_back(st);
    }
    // O; with the router folded, the router tasks (four expert rows each)
    // join the O stage on units of their own: both read only the attention
    // output and the layer input
    const bool fold = p->router_fold;
    const int n_rf = fold ? ceil_div(m->n_experts, 4) : 0;
    {
      std::vector<Task> st;
      const int o_units = n_attn_units > 0 ? n_cu - n_attn_units : n_cu;
      int nt = std::max(o_units - n_rf, ceil_div(H, rows_max(Hq * D)));
      for (auto [s0, c] : split_even(H, nt)) {
        Task t = mk_task(mk::OP_O, l);
        t.wait_b = ctr16(p->c_comb[l]);
        t.signal = ctr16(p->c_o[l]);
        t.a1 = s0; t.a2 = c;
        t.units = (uint16_t)c;
        st.push_back(t);
      }
      if (fold)
        for (auto [s0, c] : split_even(m->n_experts, n_rf)) {
          Task t = mk_task(mk::OP_ROUTER, l);
          t.flags |= mk::TF_FOLD;
          t.wait_b = ctr16(p->c_comb[l]);
          t.signal = ctr16(p->c_router[l]);
          t.a1 = s0; t.a2 = c;
          t.units = (uint16_t)c;
          st.push_back(t);
        }
      stages.push_back(st);
    }
    int n_router = 0;
    if (moe && !fold) {
      std::vector<Task> st;
      int nt = std::max(std::min(n_cu, ceil_div(m->n_experts, 8)), ceil_div(m->n_experts, rows_max(H)));
      n_router = nt;
      for (auto [s0, c] : split_even(m->n_experts, nt)) {
        Task t = mk_task(mk::OP_ROUTER, l);
        t.wait_b = ctr16(p->c_o[l]);
        t.signal = ctr16(p->c_router[l]);
        t.a1 = s0; t.a2 = c;
        t.units = (uint16_t)c;
        st.push_back(t);
      }
      stages.push_back(st);
    }
    // EXPERT: at most one per compute unit. Task i takes gate/up tile i (an
    // expert slot of one sequence and a range of FFN rows) and down tile i (a
    // range of hidden rows over every slot); its down part reads the
    // activations of every expert task of the layer. The gate/up tiles avoid
    // the units that just ran a router task (the expert tasks are dealt right
    // after the router tasks, so the last n_router expert tasks land on those
    // units): they would start their weight stream late and hold up every
    // unit's down part, whereas a down part alone waits for the activations
    // anyway.
    {
      std::vector<std::array<int, 4>> gu;  // (b, slot, f0, nf)
      const int gu_units = n_cu - n_router >= B * K ? n_cu - n_router : n_cu;
      if (moe) {
        const int per = std::max(1, gu_units / (B * K));
        for (int b = 0; b < B; ++b)
          for (int j = 0; j < K; ++j)
            for (auto [s0, c] : split_even(F, per)) gu.push_back({b, j, s0, c});
      } else {
        for (auto [s0, c] : split_even(F, n_cu)) gu.push_back({0, 0, s0, c});
      }
      std::vector<std::pair<int, int>> dn = split_even(H, n_cu);
      const size_t n = std::max(gu.size(), dn.size());
      if (n > (size_t)n_cu) {
        delete p;
        return fail(MK_EUNSUPPORTED, "mk_plan: more expert tiles than compute units");
      }
      std::vector<Task> st;
      for (size_t i = 0; i < n; ++i) {
        Task t = mk_task(mk::OP_EXPERT, l);
        t.wait_a = moe ? ctr16(p->c_router[l]) : mk::NO_CTR;
        t.wait_b = ctr16(p->c_o[l]);
        t.signal = ctr16(p->c_expert[l]);
        if (i < gu.size()) {
          t.a0 = gu[i][0]; t.aux = (uint16_t)gu[i][1]; t.a1 = gu[i][2]; t.a2 = gu[i][3];
          if (moe && gu[i][1] == 0 && gu[i][2] == 0) t.flags |= mk::TF_WRITE_TOPK;
        }
        if (fold) t.flags |= mk::TF_FOLD;
        if (i < dn.size()) t.a3 = (dn[i].first << 16) | dn[i].second;
        t.units = (uint16_t)(t.a2 + (t.a3 & 0xFFFF));
        st.push_back(t);
      }
      stages.push_back(st);
    }
  }
  // LM head (rows per tile a multiple of the streaming batch) and the final argmax merge
  if (!batch) {
    std::vector<Task> st;
    int tch = 64, cplh = 1;
    mk::gemv_map(H, &tch, &cplh);
    const int quantum = mk::gemv_groups(tch) * mk::LM_BATCH * 2;
    int rows = ceil_div(ceil_div(m->vocab, n_cu), quantum) * quantum;
    rows = std::min(rows, 2048 / quantum * quantum);
    int i = 0;
    for (int s0 = 0; s0 < m->vocab; s0 += rows) {
      Task t = mk_task(mk::OP_LM, 0);
      t.wait_b = ctr16(p->c_expert[L - 1]);
      t.signal = ctr16(p->c_lm);
      t.a1 = s0; t.a2 = std::min(rows, m->vocab - s0); t.a3 = i++;
      t.units = (uint16_t)t.a2;
      st.push_back(t);
    }
    p->n_lm = i;
    if (p->n_lm > 4096) {
      delete p;
      return fail(MK_EUNSUPPORTED, "mk_plan: more than 4096 LM-head tiles");
    }
    stages.push_back(st);
    Task f = mk_task(mk::OP_FINAL, 0);
    f.wait_b = ctr16(p->c_lm);
    f.a0 = p->n_lm;
    f.a2 = rows;  // rows per LM-head tile (the last may hold fewer)
    stages.push_back({f});
  }
  p->n_stages = (int)stages.size();

  // targets: the outputs per step of each counter's class (the sum of its
  // tasks' units); the attention splits pulled from a queue add their pages
  // (every page below the bound, per kv head); a queue counter gains one per
  // split taken and one per queue task's final, empty pull
  for (auto& st : stages)
    for (auto& t : st)
      if (t.signal != mk::NO_CTR) p->targets[t.signal] += t.units;
  uint32_t table_pages = 0;
  for (const Task& t : p->split_table) table_pages += (uint32_t)t.a3;
  if (queue)
    for (int l = 0; l < L; ++l) p->targets[p->c_attn[l * Hkv]] = table_pages;
  for (int32_t q : p->c_queue) p->targets[q] = (uint32_t)(p->split_table.size() + n_cu);
  for (auto v : p->targets)
    if (v == 0) {
      delete p;
      return fail(MK_EUNSUPPORTED, "mk_plan: counter with no producer");
    }

  // deal every stage round-robin over the units, continuing where the last
  // stage ended. A batch's attention stage (splits of ragged sequences, more
  // than one per unit, longest first) goes by pages instead: each split to
  // the unit with the fewest pages of this stage so far (ties in round-robin
  // order), so that no unit streams a fifth split while the others are done.
  p->lists.assign(n_cu, {});
  std::vector<std::vector<int>> stage_lists(n_cu);
  int cursor = 0;
  for (int s0 = 0; s0 < (int)stages.size(); ++s0) {
    const auto& st = stages[s0];
    const bool by_pages = batch && !st.empty() && st[0].op == mk::OP_ATTN && (int)st.size() > n_cu;
    if (by_pages) {
      using Load = std::pair<int64_t, int>;  // (pages so far, round-robin rank)
      std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
      for (int r = 0; r < n_cu; ++r) heap.push({0, r});
      for (const Task& t : st) {
        auto [pages, r] = heap.top();
        heap.pop();
        const int cu = (cursor + r) % n_cu;
        p->lists[cu].push_back(t);
        stage_lists[cu].push_back(s0);
        heap.push({pages + t.a3, r});
      }
    } else if (n_attn_units > 0 && !st.empty() && st[0].op != mk::OP_EXPERT && st[0].op != mk::OP_LM &&
               st[0].op != mk::OP_FINAL && (st[0].op != mk::OP_QKV || (int)st.size() == n_cu)) {
      // attention and combine on units 0 .. A-1, O and router on A .. n_cu-1,
      // QKV task i on unit i
      const bool set_a = st[0].op == mk::OP_ATTN || st[0].op == mk::OP_COMB;
      const bool all = st[0].op == mk::OP_QKV;
      const int u0 = set_a || all ? 0 : n_attn_units, nu = all ? n_cu : set_a ? n_attn_units : n_cu - n_attn_units;
      for (size_t i = 0; i < st.size(); ++i) {
        int cu = u0 + (int)(i % (size_t)nu);
        p->lists[cu].push_back(st[i]);
        stage_lists[cu].push_back(s0);
      }
      continue;
    } else {
      for (size_t i = 0; i < st.size(); ++i) {
        int cu = (cursor + (int)i) % n_cu;
        p->lists[cu].push_back(st[i]);
        stage_lists[cu].push_back(s0);
      }
    }
    cursor = (cursor + (int)st.size()) % n_cu;
  }
  // batch 1, static splits: a unit's expert task of layer l first stages the
  // first pages of the unit's next attention split (of layer l + 1, at most
  // STAGE_SCAN tasks further on) into LDS (TF_STAGE_KV)
  if (!batch && !queue) {
    for (auto& lst : p->lists)
      for (size_t i = 0; i < lst.size(); ++i) {
        if (lst[i].op != mk::OP_EXPERT) continue;
        for (size_t j = i + 1; j < lst.size() && j <= i + mk::STAGE_SCAN; ++j)
          if (lst[j].op == mk::OP_ATTN) {
            if (lst[j].layer == lst[i].layer + 1) lst[i].flags |= mk::TF_STAGE_KV;
            break;
          }
      }
  }
  if (prefill)
    for (auto& lst : p->lists)
      for (auto& t : lst)
        if (t.op == mk::OP_BQKV || t.op == mk::OP_ATTN) t.flags |= mk::TF_PREFILL;
  p->stage_of_task.clear();
  for (int cu = 0; cu < n_cu; ++cu)
    for (int s0 : stage_lists[cu]) p->stage_of_task.push_back(s0);
  p->n_tasks = p->stage_of_task.size();

  // workspace layout: tagged words (8 bytes), per layer
  {
    const int PS = D + 2;
    size_t per_layer[mk_plan::N_BUF] = {
        (size_t)B * H,                                    // XATTN
        (size_t)B * H,                                    // XFFN
        (size_t)B * Hq * D,                               // Q
        (size_t)B * Hkv * p->S_max * HG * PS,             // PART
        (size_t)B * Hq * D,                               // O
        moe ? (size_t)B * m->n_experts : 0,               // RLOG
        (size_t)B * K * F,                                // ACT
        0,                                                // LMPART (not per layer)
        (size_t)B * Hkv * 2 * D,                          // KVN
        batch && moe ? (size_t)B * K * 2 : 0,             // ROUTE
        batch ? (size_t)B * K * H : 0,                    // Y
        batch && p->o_kb > 1 ? (size_t)p->o_kb * B * H : 0,  // OPART
        batch ? (size_t)(p->q_kb - 1) * p->q_rb * B * (2 * 8 * QKV_BLOCKS + 2) : 0,   // QPART
        0};                                               // LOGIT (not per layer)
    size_t off = 0;
    for (int i = 0; i < mk_plan::N_BUF; ++i) {
      p->ws_off[i] = off;
      if (i == MK_BUF_LMPART || i == MK_BUF_LOGIT) {
        p->ws_stride[i] = 0;
        p->ws_layer_bytes[i] = i == MK_BUF_LMPART ? (size_t)p->n_lm * B * 2 * 8 : (size_t)B * m->vocab * 8;
        off = align256(off + p->ws_layer_bytes[i]);
      } else {
        p->ws_stride[i] = per_layer[i] * 8;
        p->ws_layer_bytes[i] = per_layer[i] * 8;
        off = align256(off + per_layer[i] * 8 * L);
      }
    }
    p->ws_total = off;
  }

  // device image
  {
    size_t hdr = (mk::PLAN_HDR_WORDS + n_cu + 1) * 4;
    size_t task_off = (hdr + 31) & ~size_t(31);
    const size_t split_off = task_off + p->n_tasks * sizeof(Task);
    const size_t bound_off = split_off + p->split_table.size() * sizeof(Task);
    p->image.assign(bound_off + (size_t)B * 4, 0);
    std::memcpy(p->image.data() + bound_off, p->seq_bound.data(), (size_t)B * 4);
    if (!p->split_table.empty())
      std::memcpy(p->image.data() + split_off, p->split_table.data(), p->split_table.size() * sizeof(Task));
    uint32_t* w = reinterpret_cast<uint32_t*>(p->image.data());
    w[mk::H_MAGIC] = mk::PLAN_MAGIC;
    w[mk::H_NCU] = (uint32_t)n_cu;
    w[mk::H_NTASKS] = (uint32_t)p->n_tasks;
    w[mk::H_NCTR] = (uint32_t)p->targets.size();
    w[mk::H_TASK_OFF_BYTES] = (uint32_t)task_off;
    w[mk::H_STAGES] = (uint32_t)p->n_stages;
    w[mk::H_BOUND_OFF_BYTES] = (uint32_t)bound_off;
    w[mk::H_SPLIT_OFF_BYTES] = (uint32_t)split_off;
    w[mk::H_NSPLITS] = (uint32_t)p->split_table.size();
    w[mk::H_BATCH] = (uint32_t)B;
    uint32_t* off = w + mk::PLAN_HDR_WORDS;
    Task* tasks = reinterpret_cast<Task*>(p->image.data() + task_off);
    uint32_t k = 0;
    for (int cu = 0; cu < n_cu; ++cu) {
      off[cu] = k;
      for (auto& t : p->lists[cu]) tasks[k++] = t;
    }
    off[n_cu] = k;
  }
  *out = p;
  return MK_OK;
}

extern "C" mk_status mk_plan_update(mk_plan_t* p, const int32_t* seq_lens, const int32_t* page_table,
                                    int32_t max_ctx_bound, const int32_t* ctx_bounds, int32_t* changed) {
  if (!p || !seq_lens || !page_table) return fail(MK_EINVAL, "mk_plan_update: NULL argument");
  mk_batch_desc bd;
  bd.batch = p->B;
  bd.max_pages = p->max_pages;
  bd.seq_lens = seq_lens;
  bd.page_table = page_table;
  bd.max_ctx_bound = max_ctx_bound;
  bd.ctx_bounds = ctx_bounds;
  mk_plan_t* q = nullptr;
  const mk_status st = mk_plan(&p->m, &bd, &p->opts, &q);
  if (st != MK_OK) return st;  // the plan is unchanged
  int32_t fl = 0;
  if (q->image != p->image) fl |= MK_PLAN_CHANGED_IMAGE;
  bool same_ws = q->ws_total == p->ws_total;
  for (int i = 0; i < mk_plan::N_BUF && same_ws; ++i)
    same_ws = q->ws_off[i] == p->ws_off[i] && q->ws_stride[i] == p->ws_stride[i];
  if (!same_ws) fl |= MK_PLAN_CHANGED_WORKSPACE;
  if (q->targets != p->targets || q->ctr_name != p->ctr_name) fl |= MK_PLAN_CHANGED_COUNTERS;
  // the handle keeps its identity (and a static scratch its contents and
  // epochs) unless the step must start again: the attention queue numbers
  // its pulls from the epoch and this step's item count, so a count change
  // needs fresh counters and epochs as much as a new layout does
  const uint64_t uid = (fl & (MK_PLAN_CHANGED_WORKSPACE | MK_PLAN_CHANGED_COUNTERS)) ? q->uid : p->uid;
  std::swap(*p, *q);
  p->uid = uid;
  delete q;
  if (changed) *changed = fl;
  return MK_OK;
}

// ------------------------------------------------------------------ validation

namespace {

// Output classes of the coverage check; the LM head and the final argmax sit
// in the slot of layer n_layers.
enum OutKind { K_QKV, K_ATTN, K_COMB, K_GATEUP, K_DOWN, K_O, K_ROUTER, K_TOPK, K_FFN, K_LM, K_FINAL, N_KIND };
const char* const kind_name[N_KIND] = {"qkv", "attn", "comb", "gateup", "down", "o",
                                       "router", "topk", "ffn", "lm", "final"};

// Expand the outputs a task produces into integer keys: emit(kind, key).
template <class Emit>
void task_outputs(const mk_plan_t* p, const Task& t, Emit&& emit) {
  const auto& m = p->m;
  const int D = m.head_dim, Hkv = m.n_kv_heads, Hq = m.n_q_heads;
  switch (t.op) {
    case mk::OP_QKV:
    case mk::OP_BQKV:  // the partial sums of blocks 1 .. kb-1 end in block 0's rows
      if ((t.a3 & 0xFF) != 0) break;
      for (int q = t.a1; q < t.a1 + t.a2; ++q) {
        int head, i, row;
        mk::qkv_pair(q, t.a0, p->HG, D, Hq, Hkv, &head, &i, &row);
        emit(K_QKV, row);
        emit(K_QKV, row + D / 2);
      }
      break;
    case mk::OP_ATTN:
      if (t.flags & mk::TF_QUEUE) break;  // the queue's splits are counted once per layer
      for (int pg = t.a2; pg < t.a2 + t.a3; ++pg) emit(K_ATTN, ((int64_t)t.a0 * Hkv + t.a1) * 1000000 + pg);
      break;
    case mk::OP_COMB:  // dims a2 .. a2 + a3 of heads a1, a1 + 1, .. taken as one run
      for (int d = t.a2; d < t.a2 + t.a3; ++d) emit(K_COMB, ((int64_t)t.a0 * Hq + t.a1 + d / D) * 1024 + d % D);
      break;
    case mk::OP_EXPERT: {
      const bool moe = m.n_experts > 0;
      for (int f = t.a1; f < t.a1 + t.a2; ++f) emit(K_GATEUP, moe ? ((int64_t)t.a0 * 64 + t.aux) * 1000000 + f : f);
      const int r0 = t.a3 >> 16, nr = t.a3 & 0xFFFF;
      for (int r = r0; r < r0 + nr; ++r) emit(K_DOWN, r);
      break;
    }
    case mk::OP_O:
      for (int r = t.a1; r < t.a1 + t.a2; ++r) emit(K_O, r);
      break;
    case mk::OP_BO:  // tiles of several reduction blocks publish partial sums; the sums finish rows
      if (t.a3 <= 1 || (t.flags & mk::TF_REDUCE))
        for (int r = t.a1; r < t.a1 + t.a2; ++r) emit(K_O, r);
      break;
    case mk::OP_ROUTER:  // rows a1 .. a1 + a2 of sequence a0
      for (int r = t.a1; r < t.a1 + t.a2; ++r) emit(K_ROUTER, (int64_t)t.a0 * 1000000 + r);
      break;
    case mk::OP_TOPK:  // every router row of one sequence (unless read), and its top-k
      if (!(t.flags & mk::TF_LOGITS))
        for (int r = 0; r < m.n_experts; ++r) emit(K_ROUTER, (int64_t)t.a0 * 1000000 + r);
      emit(K_TOPK, t.a0);
      break;
    case mk::OP_BEXP: {
      if (t.flags & mk::TF_SHARE) break;  // the shares cover every expert's rows once per layer
      for (int f = t.a1; f < t.a1 + t.a2; ++f) emit(K_GATEUP, (int64_t)t.a0 * 1000000 + f);
      const int r0 = t.a3 >> 16, nr = t.a3 & 0xFFFF;
      for (int r = r0; r < r0 + nr; ++r) emit(K_DOWN, (int64_t)t.a0 * 1000000 + r);
      break;
    }
    case mk::OP_BCOMB:
      for (int r = t.a1; r < t.a1 + t.a2; ++r) emit(K_FFN, (int64_t)t.a0 * 1000000 + r);
      break;
    case mk::OP_LM:
    case mk::OP_BLM:
      for (int r = t.a1; r < t.a1 + t.a2; ++r) emit(K_LM, r);
      break;
    case mk::OP_FINAL:
      emit(K_FINAL, 0);
      break;
    case mk::OP_BFINAL:
      emit(K_FINAL, t.a1);
      break;
  }
}

}  // namespace

extern "C" mk_status mk_plan_validate(const mk_plan_t* p) {
  if (!p) return fail(MK_EINVAL, "mk_plan_validate: NULL plan");
  const auto& m = p->m;
  const int L = m.n_layers, B = p->B;
  const bool moe = m.n_experts > 0;
  // expected outputs per (class, layer); the LM head and argmax at layer L
  auto slot = [L](int kind, int layer) { return (size_t)kind * (L + 1) + layer; };
  std::vector<std::vector<int64_t>> want((size_t)N_KIND * (L + 1)), got(want.size());
  for (int l = 0; l < L; ++l) {
    auto w = [&](int kind) -> std::vector<int64_t>& { return want[slot(kind, l)]; };
    for (int r = 0; r < p->QKV_ROWS; ++r) w(K_QKV).push_back(r);
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < m.n_kv_heads; ++g)
        for (int pg = 0; pg < ((p->batch ? p->seq_bound[b] : p->bound) + 15) / 16; ++pg)
          w(K_ATTN).push_back(((int64_t)b * m.n_kv_heads + g) * 1000000 + pg);
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < m.n_q_heads; ++h)
        for (int d = 0; d < m.head_dim; ++d) w(K_COMB).push_back(((int64_t)b * m.n_q_heads + h) * 1024 + d);
    for (int r = 0; r < m.hidden; ++r) w(K_O).push_back(r);
    if (p->batch) {
      const int NE = moe ? m.n_experts : 1;
      if (moe)
        for (int b = 0; b < B; ++b) {
          for (int r = 0; r < m.n_experts; ++r) w(K_ROUTER).push_back((int64_t)b * 1000000 + r);
          w(K_TOPK).push_back(b);
        }
      for (int e = 0; e < NE; ++e) {
        for (int f = 0; f < p->F; ++f) w(K_GATEUP).push_back((int64_t)e * 1000000 + f);
        for (int r = 0; r < m.hidden; ++r) w(K_DOWN).push_back((int64_t)e * 1000000 + r);
      }
      for (int b = 0; b < B; ++b)
        for (int r = 0; r < m.hidden; ++r) w(K_FFN).push_back((int64_t)b * 1000000 + r);
      continue;
    }
    for (int r = 0; r < m.hidden; ++r) w(K_DOWN).push_back(r);
    if (moe) {
      for (int r = 0; r < m.n_experts; ++r) w(K_ROUTER).push_back(r);
      for (int b = 0; b < B; ++b)
        for (int j = 0; j < m.top_k; ++j)
          for (int f = 0; f < p->F; ++f) w(K_GATEUP).push_back(((int64_t)b * 64 + j) * 1000000 + f);
    } else {
      for (int f = 0; f < p->F; ++f) w(K_GATEUP).push_back(f);
    }
  }
  for (int r = 0; r < m.vocab; ++r) want[slot(K_LM, L)].push_back(r);
  for (int b = 0; b < (p->batch ? B : 1); ++b) want[slot(K_FINAL, L)].push_back(b);

  std::vector<uint32_t> producers(p->targets.size(), 0);
  std::vector<int> ctr_stage(p->targets.size(), -1);
  size_t k = 0;
  for (int cu = 0; cu < p->n_cu; ++cu) {
    int last = -1;
    std::set<int> expert_layers;
    for (auto& t : p->lists[cu]) {
      int st = p->stage_of_task[k++];
      if (st < last) return fail(MK_EINVAL, "validate: list of unit " + std::to_string(cu) + " is not in stage order");
      last = st;
      if ((t.op == mk::OP_EXPERT || t.op == mk::OP_BEXP) && !expert_layers.insert(t.layer).second)
        return fail(MK_EINVAL, "validate: unit " + std::to_string(cu) + " holds two expert tasks of layer " +
                                   std::to_string(t.layer) + " (their down parts would wait on each other)");
      if (t.layer >= L && t.op != mk::OP_LM && t.op != mk::OP_BLM && t.op != mk::OP_FINAL && t.op != mk::OP_BFINAL)
        return fail(MK_EINVAL, "validate: task of layer " + std::to_string(t.layer) + " beyond the model");
      const int tl = (t.op == mk::OP_LM || t.op == mk::OP_BLM || t.op == mk::OP_FINAL || t.op == mk::OP_BFINAL)
                         ? L : t.layer;
      task_outputs(p, t, [&](int kind, int64_t v) { got[slot(kind, tl)].push_back(v); });
      if (t.signal != mk::NO_CTR) {
        if (t.signal >= p->targets.size()) return fail(MK_EINVAL, "validate: signal counter out of range");
        producers[t.signal] += t.units;
        if (ctr_stage[t.signal] >= 0 && ctr_stage[t.signal] != st)
          return fail(MK_EINVAL, "validate: counter signalled from two stages");
        ctr_stage[t.signal] = st;
      }
    }
  }
  if (p->expert_share)  // the expert shares of a layer cover every expert's rows once
    for (int l = 0; l < L; ++l)
      for (int e = 0; e < m.n_experts; ++e) {
        for (int f = 0; f < p->F; ++f) got[slot(K_GATEUP, l)].push_back((int64_t)e * 1000000 + f);
        for (int r = 0; r < m.hidden; ++r) got[slot(K_DOWN, l)].push_back((int64_t)e * 1000000 + r);
      }
  if (p->attn_queue)  // every split of the queue's table, once per layer
    for (int l = 0; l < L; ++l)
      for (const Task& t : p->split_table)
        for (int pg = t.a2; pg < t.a2 + t.a3; ++pg)
          got[slot(K_ATTN, l)].push_back(((int64_t)t.a0 * m.n_kv_heads + t.a1) * 1000000 + pg);
  // every expected output exactly once, nothing else
  for (size_t i = 0; i < want.size(); ++i) {
    auto& a = want[i];
    auto& b = got[i];
    std::sort(a.begin(), a.end());
    std::sort(b.begin(), b.end());
    if (a != b) {
      const int kind = (int)(i / (L + 1)), layer = (int)(i % (L + 1));
      const std::string key = std::string(kind_name[kind]) + (layer < L ? ":" + std::to_string(layer) : "");
      if (b.empty()) return fail(MK_EINVAL, "validate: no task covers " + key);
      if (a.empty()) return fail(MK_EINVAL, "validate: tasks of an unexpected kind (" + key + ")");
      return fail(MK_EINVAL, "validate: outputs of " + key + " not covered exactly once");
    }
  }
  // a counter's target is the outputs its tasks produce per step (the
  // attention splits of a queue add their pages on the device: every page
  // below the bound, per kv head)
  std::set<int32_t> queues(p->c_queue.begin(), p->c_queue.end());
  uint32_t table_pages = 0;
  for (const Task& t : p->split_table) table_pages += (uint32_t)t.a3;
  if (p->attn_queue)
    for (int l = 0; l < L; ++l) producers[p->c_attn[l * m.n_kv_heads]] += table_pages;
  for (size_t c = 0; c < p->targets.size(); ++c)
    if (!queues.count((int32_t)c) && producers[c] != p->targets[c])
      return fail(MK_EINVAL, "validate: counter " + p->ctr_name[c] + " target != the outputs of its tasks");
  k = 0;
  for (int cu = 0; cu < p->n_cu; ++cu)
    for (auto& t : p->lists[cu]) {
      int st = p->stage_of_task[k++];
      for (uint16_t w : {t.wait_a, t.wait_b}) {
        if (w == mk::NO_CTR) continue;
        if (w >= p->targets.size()) return fail(MK_EINVAL, "validate: wait counter out of range");
        if (ctr_stage[w] >= st) return fail(MK_EINVAL, "validate: task waits on a counter of its own or a later stage");
      }
      if (t.signal == mk::NO_CTR && t.units != 0) return fail(MK_EINVAL, "validate: units without a counter");
    }
  return MK_OK;
}

// ------------------------------------------------------------------ simulation

// Runs the per-unit lists on n_cu virtual units under seeded random
// interleavings, modelling the waits the device performs: a task starts only
// once every task producing data it reads has finished (the device polls the
// tagged words themselves; here the producers of a word are taken by class,
// a superset of the words a task reads, so a deadlock on the device is a
// deadlock here). Two-phase tasks: an expert task first publishes its gate/up
// activations, then its down part waits until every expert task of its layer
// has published. A unit runs its list in order, one task at a time. Every
// run must finish (no deadlock) with every counter at epoch x target.
extern "C" mk_status mk_plan_simulate(const mk_plan_t* p, uint64_t seed, int32_t n_runs) {
  if (!p || n_runs <= 0) return fail(MK_EINVAL, "mk_plan_simulate: bad args");
  const auto& m = p->m;
  const int L = m.n_layers, Hkv = m.n_kv_heads, HG = p->HG;
  const bool moe = m.n_experts > 0;
  std::mt19937_64 rng(seed);
  std::vector<uint64_t> ctr(p->targets.size(), 0);
  // task kinds: the op, or a kind of its own for the partial sums of a split
  // reduction (batch QKV / O blocks 1 ..), which block 0 reads
  constexpr int K_QPART = mk::OP_COUNT, K_OPART = mk::OP_COUNT + 1, N_KIND = mk::OP_COUNT + 2;
  auto kind = [](const Task& t) -> int {
    if (t.op == mk::OP_BQKV && (t.a3 & 0xFF) != 0) return K_QPART;
    if (t.op == mk::OP_BO && t.a3 > 1 && !(t.flags & mk::TF_REDUCE)) return K_OPART;
    return t.op;
  };
  auto slot = [&](int k, int l, int g) { return ((size_t)k * (L + 1) + l) * (Hkv + 1) + g; };
  const size_t n_slots = (size_t)N_KIND * (L + 1) * (Hkv + 1);
  std::vector<uint32_t> total(n_slots, 0);
  auto group_of = [&](const Task& t) -> int {  // kv group of a QKV or attention task, Hkv: any
    if (t.op == mk::OP_ATTN) return (t.flags & mk::TF_QUEUE) ? Hkv : t.a1;
    if (t.op == mk::OP_QKV || t.op == mk::OP_BQKV) return t.a0;
    return Hkv;
  };
  for (int cu = 0; cu < p->n_cu; ++cu)
    for (auto& t : p->lists[cu]) {
      total[slot(kind(t), t.layer, Hkv)]++;
      const int g = group_of(t);
      if (t.op == mk::OP_ATTN && g == Hkv) {
        for (int gg = 0; gg < Hkv; ++gg) total[slot(kind(t), t.layer, gg)]++;
      } else if (g < Hkv) {
        total[slot(kind(t), t.layer, g)]++;
      }
    }
  const int qkv_op = p->batch ? mk::OP_BQKV : mk::OP_QKV;
  auto two_phase = [](int op) { return op == mk::OP_EXPERT || op == mk::OP_BEXP; };
  for (int run = 0; run < n_runs; ++run) {
    const uint64_t epoch = (uint64_t)run + 1;
    std::vector<uint32_t> done(n_slots, 0);
    std::vector<uint32_t> published(L, 0);      // expert gate/up parts finished per layer
    std::vector<size_t> head(p->n_cu, 0);
    std::vector<char> phase(p->n_cu, 0);        // expert task at the head: 1 = published
    auto all_done = [&](int k, int l, int g) { return done[slot(k, l, g)] == total[slot(k, l, g)]; };
    // the data a task reads: complete when every producer (by class) finished
    auto inputs_ok = [&](const Task& t) -> bool {
      const int l = t.layer;
      const int ffn_op = p->batch ? mk::OP_BCOMB : mk::OP_EXPERT;
      switch (kind(t)) {
        case mk::OP_QKV: return l == 0 || all_done(ffn_op, l - 1, Hkv);
        case mk::OP_ATTN: return all_done(qkv_op, l, group_of(t));
        case mk::OP_COMB: return all_done(mk::OP_ATTN, l, t.a1 / HG);
        case mk::OP_O: return all_done(mk::OP_COMB, l, Hkv);
        case mk::OP_ROUTER:
          if (t.flags & mk::TF_FOLD) return all_done(mk::OP_COMB, l, Hkv) && (l == 0 || all_done(ffn_op, l - 1, Hkv));
          return all_done(p->batch ? mk::OP_BO : mk::OP_O, l, Hkv);
        case mk::OP_EXPERT: return all_done(mk::OP_O, l, Hkv) && (!moe || all_done(mk::OP_ROUTER, l, Hkv));
        case mk::OP_LM: return all_done(mk::OP_EXPERT, L - 1, Hkv);
        case mk::OP_FINAL: return all_done(mk::OP_LM, 0, Hkv);
        case K_QPART: return l == 0 || all_done(ffn_op, l - 1, Hkv);
        case mk::OP_BQKV:
          return (l == 0 || all_done(ffn_op, l - 1, Hkv)) && all_done(K_QPART, l, Hkv);
        case K_OPART: return all_done(mk::OP_COMB, l, Hkv);
        case mk::OP_BO: return all_done(mk::OP_COMB, l, Hkv) && all_done(K_OPART, l, Hkv);
        case mk::OP_TOPK:
          return all_done(mk::OP_BO, l, Hkv) && (!(t.flags & mk::TF_LOGITS) || all_done(mk::OP_ROUTER, l, Hkv));
        case mk::OP_BEXP: return all_done(mk::OP_BO, l, Hkv) && (!moe || all_done(mk::OP_TOPK, l, Hkv));
        case mk::OP_BCOMB: return all_done(mk::OP_BEXP, l, Hkv) && (!moe || all_done(mk::OP_TOPK, l, Hkv));
        case mk::OP_BLM: return all_done(mk::OP_BCOMB, L - 1, Hkv);
        case mk::OP_BFINAL: return all_done(mk::OP_BLM, 0, Hkv);
      }
      return false;
    };
    size_t remaining = p->n_tasks;
    std::vector<int> runnable;
    while (remaining) {
      runnable.clear();
      for (int cu = 0; cu < p->n_cu; ++cu) {
        if (head[cu] >= p->lists[cu].size()) continue;
        const Task& t = p->lists[cu][head[cu]];
        if (two_phase(t.op) && phase[cu] == 1) {
          if (published[t.layer] == total[slot(t.op, t.layer, Hkv)]) runnable.push_back(cu);
        } else if (inputs_ok(t)) {
          runnable.push_back(cu);
        }
      }
      if (runnable.empty()) {
        std::string msg = "simulate: deadlock in epoch " + std::to_string(epoch) + "; blocked:";
        int shown = 0;
        for (int cu = 0; cu < p->n_cu && shown < 8; ++cu)
          if (head[cu] < p->lists[cu].size()) {
            const Task& t = p->lists[cu][head[cu]];
            msg += " unit " + std::to_string(cu) + " op " + std::to_string(t.op) + " layer " +
                   std::to_string(t.layer) + " reads " +
                   (t.wait_b != mk::NO_CTR ? p->ctr_name[t.wait_b] : std::string("-"));
            ++shown;
          }
        return fail(MK_ESTATE, msg);
      }
      // advance a random subset of runnable units by one event each, in random order
      std::shuffle(runnable.begin(), runnable.end(), rng);
      size_t n = 1 + rng() % runnable.size();
      for (size_t i = 0; i < n; ++i) {
        int cu = runnable[i];
        const Task& t = p->lists[cu][head[cu]];
        if (two_phase(t.op) && phase[cu] == 0) {
          phase[cu] = 1;
          published[t.layer]++;
          continue;
        }
        phase[cu] = 0;
        head[cu]++;
        remaining--;
        done[slot(kind(t), t.layer, Hkv)]++;
        const int g = group_of(t);
        if (t.op == mk::OP_ATTN && g == Hkv) {
          for (int gg = 0; gg < Hkv; ++gg) done[slot(kind(t), t.layer, gg)]++;
        } else if (g < Hkv) {
          done[slot(kind(t), t.layer, g)]++;
        }
        if (t.signal != mk::NO_CTR) ctr[t.signal] += t.units;
      }
    }
    // the queue tasks' pulls, and the pages of the splits they took
    for (int32_t q : p->c_queue) ctr[q] += p->targets[q];
    if (p->attn_queue)
      for (int l = 0; l < L; ++l) ctr[p->c_attn[l * Hkv]] += p->targets[p->c_attn[l * Hkv]];
    for (size_t c = 0; c < ctr.size(); ++c)
      if (ctr[c] != epoch * p->targets[c])
        return fail(MK_ESTATE, "simulate: counter " + p->ctr_name[c] + " ends epoch off target");
  }
  return MK_OK;
}

// ------------------------------------------------------------------ accessors

extern "C" size_t mk_plan_device_bytes(const mk_plan_t* p) { return p ? p->image.size() : 0; }
extern "C" size_t mk_plan_workspace_bytes(const mk_plan_t* p) { return p ? p->ws_total : 0; }
extern "C" size_t mk_plan_counter_bytes(const mk_plan_t* p) {
  return p ? p->targets.size() * mk::CTR_LINES * mk::CTR_STRIDE * 4 : 0;
}
extern "C" int32_t mk_plan_n_tasks(const mk_plan_t* p) { return p ? (int32_t)p->n_tasks : -1; }
extern "C" int32_t mk_plan_n_counters(const mk_plan_t* p) { return p ? (int32_t)p->targets.size() : -1; }
extern "C" int32_t mk_plan_n_cu(const mk_plan_t* p) { return p ? p->n_cu : -1; }

extern "C" mk_status mk_plan_export(const mk_plan_t* p, void* buf, size_t bytes) {
  if (!p || !buf) return fail(MK_EINVAL, "mk_plan_export: NULL argument");
  if (bytes < p->image.size()) return fail(MK_EINVAL, "mk_plan_export: buffer too small");
  std::memcpy(buf, p->image.data(), p->image.size());
  return MK_OK;
}

extern "C" mk_status mk_plan_buffer(const mk_plan_t* p, int32_t which, int32_t layer, size_t* off,
                                    size_t* bytes) {
  if (!p || !off || !bytes || which < 0 || which >= mk_plan::N_BUF)
    return fail(MK_EINVAL, "mk_plan_buffer: bad args");
  const bool per_layer = which != MK_BUF_LMPART && which != MK_BUF_LOGIT;
  if (per_layer && (layer < 0 || layer >= p->m.n_layers)) return fail(MK_EINVAL, "mk_plan_buffer: bad layer");
  *off = p->ws_off[which] + (per_layer ? (size_t)layer * p->ws_stride[which] : 0);
  *bytes = p->ws_layer_bytes[which];
  return MK_OK;
}

extern "C" const char* mk_plan_counter_name(const mk_plan_t* p, int32_t i) {
  if (!p || i < 0 || i >= (int32_t)p->ctr_name.size()) {
    fail(MK_EINVAL, "mk_plan_counter_name: no such counter");
    return nullptr;
  }
  return p->ctr_name[i].c_str();
}

extern "C" mk_status mk_plan_counter_targets(const mk_plan_t* p, uint32_t* out, int32_t n) {
  if (!p || !out || n < (int32_t)p->targets.size()) return fail(MK_EINVAL, "mk_plan_counter_targets: bad args");
  std::copy(p->targets.begin(), p->targets.end(), out);
  return MK_OK;
}

extern "C" void mk_plan_free(mk_plan_t* p) { delete p; }
