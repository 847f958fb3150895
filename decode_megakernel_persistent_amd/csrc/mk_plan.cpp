// Host planner: decomposes one decode step into tile tasks, deals them over
// the compute units, allocates dependency counters, lays out the workspace,
// and checks the result (validate) or executes it on virtual compute units
// (simulate). Pure host code: no device is touched (kern page, "The runtime":
// state decisions made as pure host code are tested without a GPU).
//
// The decomposition follows the megakernel page ("What is a Megakernel?" and
// the caption of Image 2): every operation of the step is cut into tiles, one
// task per tile; the host deals the tasks round-robin over the compute units
// so each unit gets its own list in device memory; counters express which
// producers a task waits for. Stages, in order, per layer:
//   QKV (per kv group: q, k, v rows of the group, rotary epilogue, KV append)
//   ATTN (per sequence, kv group and page range: split-KV partials)
//   COMB (per sequence and query head: log-sum-exp merge of the splits)
//   O    (rows of W_o, residual)
//   ROUTER (MoE: rows of W_router)
//   GATEUP (MoE: per sequence, expert slot and row range; dense: row range)
//   DOWN (rows of W_down, weighted combine over slots, residual)
// then LM (rows of the LM head, local argmax) and FINAL (argmax merge).
#include <algorithm>
#include <cstring>
#include <map>
#include <numeric>
#include <random>
#include <set>
#include <string>
#include <tuple>
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

int rows_cap(int K, int B, int mult) {
  int tc = 0, cpl = 0;
  mk::gemv_map(K, &tc, &cpl);
  int per = std::max(1, tc / 64) * std::max(1, B) * std::max(1, mult);
  return std::max(1, mk::GEMV_LDS_FLOATS / per);
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
  int tc, cpl;
  for (int K : {H, Hq * D, F})
    if (!mk::gemv_map(K, &tc, &cpl))
      return fail(MK_EUNSUPPORTED, "mk_plan: reduction width " + std::to_string(K) +
                                       " has no GEMV mapping (need a multiple of 256)");
  {
    int tcf = 64, cplf = 1;
    mk::gemv_map(F, &tcf, &cplf);
    int kk = moe ? m->top_k : 1;
    if ((mk::NT / tcf) % kk)
      return fail(MK_EUNSUPPORTED, "mk_plan: down-projection mapping needs top_k to divide " +
                                       std::to_string(mk::NT / tcf));
  }
  const int B = bd->batch;
  if (B != 1) return fail(MK_EUNSUPPORTED, "mk_plan: only batch 1 is implemented by the kernels");
  if (!bd->seq_lens || !bd->page_table || bd->max_pages <= 0)
    return fail(MK_EINVAL, "mk_plan: seq_lens / page_table / max_pages missing");
  const int bound = bd->max_ctx_bound;
  const int pg_bound = (bound + 15) / 16;
  if (bound <= 0 || pg_bound > bd->max_pages)
    return fail(MK_EBOUNDS, "mk_plan: max_ctx_bound needs " + std::to_string(pg_bound) +
                                " pages per sequence, page table has " + std::to_string(bd->max_pages));
  for (int b = 0; b < B; ++b) {
    if (bd->seq_lens[b] < 0 || bd->seq_lens[b] + 1 > bound)
      return fail(MK_EBOUNDS, "mk_plan: seq_lens[" + std::to_string(b) + "] + 1 exceeds max_ctx_bound");
    for (int j = 0; j < pg_bound; ++j)
      if (bd->page_table[(int64_t)b * bd->max_pages + j] < 0)
        return fail(MK_EBOUNDS, "mk_plan: sequence " + std::to_string(b) +
                                    " has no page mapped at logical page " + std::to_string(j));
  }
  int n_cu = o && o->n_cu > 0 ? o->n_cu : 0;
  if (n_cu == 0) {
    if (mk_device_cu_count(&n_cu) != MK_OK || n_cu <= 0)
      return fail(MK_EINVAL, "mk_plan: opts.n_cu is 0 and no device could be queried");
  }
  if (n_cu > 4096) return fail(MK_EINVAL, "mk_plan: n_cu too large");

  auto* p = new mk_plan_t();
  p->m = *m;
  p->B = B;
  p->max_pages = bd->max_pages;
  p->bound = bound;
  p->n_cu = n_cu;
  p->seq_lens.assign(bd->seq_lens, bd->seq_lens + B);
  p->page_table.assign(bd->page_table, bd->page_table + (int64_t)B * bd->max_pages);
  p->HG = Hq / Hkv;
  p->QKV_ROWS = (Hq + 2 * Hkv) * D;
  p->F = F;
  p->n_pairs_g = (p->HG * D + 2 * D) / 2;
  const int HG = p->HG, K = moe ? m->top_k : 1;

  auto new_ctr = [&](const std::string& name) {
    p->targets.push_back(0);
    p->ctr_name.push_back(name);
    return (int32_t)p->targets.size() - 1;
  };
  for (int l = 0; l < L; ++l) {
    for (int g = 0; g < Hkv; ++g) p->c_qkv.push_back(new_ctr("qkv[" + std::to_string(l) + "][" + std::to_string(g) + "]"));
    for (int g = 0; g < Hkv; ++g) p->c_attn.push_back(new_ctr("attn[" + std::to_string(l) + "][" + std::to_string(g) + "]"));
    p->c_comb.push_back(new_ctr("comb[" + std::to_string(l) + "]"));
    p->c_o.push_back(new_ctr("o[" + std::to_string(l) + "]"));
    p->c_router.push_back(moe ? new_ctr("router[" + std::to_string(l) + "]") : -1);
    p->c_gateup.push_back(new_ctr("gateup[" + std::to_string(l) + "]"));
    p->c_down.push_back(new_ctr("down[" + std::to_string(l) + "]"));
  }
  p->c_lm = new_ctr("lm");
  if (p->targets.size() >= mk::NO_CTR) {
    delete p;
    return fail(MK_EUNSUPPORTED, "mk_plan: too many counters");
  }

  // attention splits: pages per split chosen so the step has about n_cu split tasks
  const int pg_total = pg_bound * B * Hkv;
  int pps = o && o->attn_split_pages > 0 ? o->attn_split_pages : (pg_total + n_cu - 1) / n_cu;
  pps = std::max(std::max(1, pps), (pg_bound + 1023) / 1024);  // at most 1024 splits per (b, g)
  p->n_split.assign(B, 0);
  for (int b = 0; b < B; ++b) p->n_split[b] = (pg_bound + pps - 1) / pps;
  p->S_max = *std::max_element(p->n_split.begin(), p->n_split.end());

  std::vector<std::vector<Task>> stages;
  auto ctr16 = [](int c) { return c < 0 ? mk::NO_CTR : (uint16_t)c; };
  for (int l = 0; l < L; ++l) {
    // QKV: tiles of rotary pairs within one kv group
    {
      std::vector<Task> st;
      int per_g = std::max(1, n_cu / Hkv);
      int cap_pairs = std::max(1, rows_cap(H, B, 1) / 2);
      per_g = std::max(per_g, (p->n_pairs_g + cap_pairs - 1) / cap_pairs);
      for (int g = 0; g < Hkv; ++g)
        for (auto [s, c] : split_even(p->n_pairs_g, per_g)) {
          Task t = mk_task(mk::OP_QKV, l);
          t.wait_b = l == 0 ? mk::NO_CTR : ctr16(p->c_down[l - 1]);
          t.signal = ctr16(p->c_qkv[l * Hkv + g]);
          t.a0 = g; t.a1 = s; t.a2 = c;
          st.push_back(t);
        }
      stages.push_back(st);
    }
    // ATTN: split-KV tasks per (b, g)
    {
      std::vector<Task> st;
      for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g) {
          int si = 0;
          for (auto [s, c] : split_even(pg_bound, p->n_split[b])) {
            Task t = mk_task(mk::OP_ATTN, l);
            t.wait_b = ctr16(p->c_qkv[l * Hkv + g]);
            t.signal = ctr16(p->c_attn[l * Hkv + g]);
            t.a0 = b; t.a1 = g; t.a2 = s; t.a3 = c; t.aux = (uint16_t)si++;
            st.push_back(t);
          }
        }
      stages.push_back(st);
    }
    // COMB: one query head of one sequence per task
    {
      std::vector<Task> st;
      for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
          Task t = mk_task(mk::OP_COMB, l);
          t.wait_b = ctr16(p->c_attn[l * Hkv + h / HG]);
          t.signal = ctr16(p->c_comb[l]);
          t.a0 = b; t.a1 = h; t.a2 = 1; t.a3 = p->n_split[b];
          st.push_back(t);
        }
      stages.push_back(st);
    }
    // O
    {
      std::vector<Task> st;
      int nt = std::max(n_cu, (H + rows_cap(Hq * D, B, 1) - 1) / rows_cap(Hq * D, B, 1));
      for (auto [s, c] : split_even(H, nt)) {
        Task t = mk_task(mk::OP_O, l);
        t.wait_b = ctr16(p->c_comb[l]);
        t.signal = ctr16(p->c_o[l]);
        t.a1 = s; t.a2 = c;
        st.push_back(t);
      }
      stages.push_back(st);
    }
    if (moe) {
      std::vector<Task> st;
      for (auto [s, c] : split_even(m->n_experts, std::max(1, n_cu / 4))) {
        Task t = mk_task(mk::OP_ROUTER, l);
        t.wait_b = ctr16(p->c_o[l]);
        t.signal = ctr16(p->c_router[l]);
        t.a1 = s; t.a2 = c;
        st.push_back(t);
      }
      stages.push_back(st);
    }
    // GATEUP
    {
      std::vector<Task> st;
      int cap = std::max(1, rows_cap(H, moe ? 1 : B, 2));
      if (moe) {
        int per = std::max(1, n_cu / (B * K));
        per = std::max(per, (F + cap - 1) / cap);
        for (int b = 0; b < B; ++b)
          for (int j = 0; j < K; ++j) {
            bool first = true;
            for (auto [s, c] : split_even(F, per)) {
              Task t = mk_task(mk::OP_GATEUP, l);
              t.wait_a = ctr16(p->c_router[l]);
              t.signal = ctr16(p->c_gateup[l]);
              t.a0 = b; t.aux = (uint16_t)j; t.a1 = s; t.a2 = c;
              if (first && j == 0) t.flags |= mk::TF_WRITE_TOPK;
              first = false;
              st.push_back(t);
            }
          }
      } else {
        int per = std::max(n_cu, (F + cap - 1) / cap);
        for (auto [s, c] : split_even(F, per)) {
          Task t = mk_task(mk::OP_GATEUP, l);
          t.wait_b = ctr16(p->c_o[l]);
          t.signal = ctr16(p->c_gateup[l]);
          t.a0 = -1; t.a1 = s; t.a2 = c;
          st.push_back(t);
        }
      }
      stages.push_back(st);
    }
    // DOWN
    {
      std::vector<Task> st;
      int cap = rows_cap(F, B, K);
      int nt = std::max(n_cu, (H + cap - 1) / cap);
      for (auto [s, c] : split_even(H, nt)) {
        Task t = mk_task(mk::OP_DOWN, l);
        t.wait_a = moe ? ctr16(p->c_router[l]) : mk::NO_CTR;
        t.wait_b = ctr16(p->c_gateup[l]);
        t.signal = ctr16(p->c_down[l]);
        t.a1 = s; t.a2 = c;
        st.push_back(t);
      }
      stages.push_back(st);
    }
  }
  // LM head and final argmax merge
  {
    std::vector<Task> st;
    int cap = std::min(1024, rows_cap(H, B, 1));
    int nt = std::max(n_cu, (m->vocab + cap - 1) / cap);
    int i = 0;
    for (auto [s, c] : split_even(m->vocab, nt)) {
      Task t = mk_task(mk::OP_LM, 0);
      t.wait_b = ctr16(p->c_down[L - 1]);
      t.signal = ctr16(p->c_lm);
      t.a1 = s; t.a2 = c; t.a3 = i++;
      st.push_back(t);
    }
    p->n_lm = i;
    stages.push_back(st);
    Task f = mk_task(mk::OP_FINAL, 0);
    f.wait_b = ctr16(p->c_lm);
    f.a0 = p->n_lm;
    stages.push_back({f});
  }
  p->n_stages = (int)stages.size();

  // GEMV thread mapping per task kind (log2 TC in the high nibble of flags)
  auto lg = [](int v) { int r = 0; while ((1 << r) < v) ++r; return r; };
  for (auto& st : stages)
    for (auto& t : st) {
      int K = 0;
      switch (t.op) {
        case mk::OP_QKV: case mk::OP_ROUTER: case mk::OP_GATEUP: case mk::OP_LM: K = H; break;
        case mk::OP_O: K = Hq * D; break;
        case mk::OP_DOWN: K = F; break;
        default: break;
      }
      if (K) {
        int tcK = 0, cplK = 0;
        mk::gemv_map(K, &tcK, &cplK);
        t.flags = (uint8_t)((t.flags & 0x0F) | (lg(tcK) << 4));
      }
    }

  // producer counts -> targets, then the per-epoch counts carried by the waits
  for (auto& st : stages)
    for (auto& t : st)
      if (t.signal != mk::NO_CTR) p->targets[t.signal]++;
  for (auto& st : stages)
    for (auto& t : st) {
      if (t.wait_a != mk::NO_CTR) t.cnt_a = (uint16_t)p->targets[t.wait_a];
      if (t.wait_b != mk::NO_CTR) t.cnt_b = (uint16_t)p->targets[t.wait_b];
    }
  for (auto v : p->targets)
    if (v == 0 || v > 65535) {
      delete p;
      return fail(MK_EUNSUPPORTED, "mk_plan: counter with 0 or > 65535 producers");
    }

  // deal every stage round-robin over the units, continuing where the last stage ended
  p->lists.assign(n_cu, {});
  std::vector<std::vector<int>> stage_lists(n_cu);
  int cursor = 0;
  for (int s = 0; s < (int)stages.size(); ++s) {
    for (size_t i = 0; i < stages[s].size(); ++i) {
      int cu = (cursor + (int)i) % n_cu;
      p->lists[cu].push_back(stages[s][i]);
      stage_lists[cu].push_back(s);
    }
    cursor = (cursor + (int)stages[s].size()) % n_cu;
  }
  p->stage_of_task.clear();
  for (int cu = 0; cu < n_cu; ++cu)
    for (int s : stage_lists[cu]) p->stage_of_task.push_back(s);
  p->n_tasks = p->stage_of_task.size();

  // workspace layout
  {
    const int PS = D + 4;
    size_t per_layer[8] = {
        (size_t)B * H * 4,                       // XATTN
        (size_t)B * H * 4,                       // XFFN
        (size_t)B * Hq * D * 4,                  // Q
        (size_t)B * Hq * p->S_max * PS * 4,      // PART
        (size_t)B * Hq * D * 4,                  // O
        moe ? (size_t)B * m->n_experts * 4 : 0,  // RLOG
        (size_t)B * K * F * 4,                   // ACT
        0};
    size_t off = 0;
    for (int i = 0; i < 7; ++i) {
      p->ws_off[i] = off;
      p->ws_stride[i] = per_layer[i];
      p->ws_layer_bytes[i] = per_layer[i];
      off = align256(off + per_layer[i] * L);
    }
    p->ws_off[7] = off;
    p->ws_stride[7] = 0;
    p->ws_layer_bytes[7] = (size_t)p->n_lm * B * 8;
    off = align256(off + p->ws_layer_bytes[7]);
    p->ws_total = off;
  }

  // device image
  {
    size_t hdr = (mk::PLAN_HDR_WORDS + n_cu + 1) * 4;
    size_t task_off = (hdr + 31) & ~size_t(31);
    p->image.assign(task_off + p->n_tasks * sizeof(Task), 0);
    uint32_t* w = reinterpret_cast<uint32_t*>(p->image.data());
    w[mk::H_MAGIC] = mk::PLAN_MAGIC;
    w[mk::H_NCU] = (uint32_t)n_cu;
    w[mk::H_NTASKS] = (uint32_t)p->n_tasks;
    w[mk::H_NCTR] = (uint32_t)p->targets.size();
    w[mk::H_TASK_OFF_BYTES] = (uint32_t)task_off;
    w[mk::H_STAGES] = (uint32_t)p->n_stages;
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

// ------------------------------------------------------------------ validation

namespace {

struct Cover {
  std::string what;
  std::vector<int64_t> items;
};

// Expand the outputs a task produces into integer keys per (op, layer).
void task_outputs(const mk_plan_t* p, const Task& t, std::vector<std::pair<std::string, int64_t>>& out) {
  const auto& m = p->m;
  const int D = m.head_dim, Hkv = m.n_kv_heads, Hq = m.n_q_heads;
  std::string key = std::to_string(t.op) + ":" + std::to_string(t.layer);
  switch (t.op) {
    case mk::OP_QKV:
      for (int q = t.a1; q < t.a1 + t.a2; ++q) {
        int head, i, row;
        mk::qkv_pair(q, t.a0, p->HG, D, Hq, Hkv, &head, &i, &row);
        out.push_back({key, row});
        out.push_back({key, row + D / 2});
      }
      break;
    case mk::OP_ATTN:
      for (int pg = t.a2; pg < t.a2 + t.a3; ++pg)
        out.push_back({key, ((int64_t)t.a0 * Hkv + t.a1) * 1000000 + pg});
      break;
    case mk::OP_COMB:
      for (int h = t.a1; h < t.a1 + t.a2; ++h) out.push_back({key, (int64_t)t.a0 * Hq + h});
      break;
    case mk::OP_GATEUP:
      for (int f = t.a1; f < t.a1 + t.a2; ++f)
        out.push_back({key, t.a0 < 0 ? f : ((int64_t)t.a0 * 64 + t.aux) * 1000000 + f});
      break;
    case mk::OP_O: case mk::OP_ROUTER: case mk::OP_DOWN: case mk::OP_LM:
      for (int r = t.a1; r < t.a1 + t.a2; ++r) out.push_back({key, r});
      break;
    case mk::OP_FINAL:
      out.push_back({key, 0});
      break;
  }
}

}  // namespace

extern "C" mk_status mk_plan_validate(const mk_plan_t* p) {
  if (!p) return fail(MK_EINVAL, "mk_plan_validate: NULL plan");
  const auto& m = p->m;
  const int L = m.n_layers, B = p->B;
  const bool moe = m.n_experts > 0;
  // expected output sets
  std::map<std::string, std::set<int64_t>> want;
  for (int l = 0; l < L; ++l) {
    auto k = [&](int op) { return std::to_string(op) + ":" + std::to_string(l); };
    for (int r = 0; r < p->QKV_ROWS; ++r) want[k(mk::OP_QKV)].insert(r);
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < m.n_kv_heads; ++g)
        for (int pg = 0; pg < (p->bound + 15) / 16; ++pg)
          want[k(mk::OP_ATTN)].insert(((int64_t)b * m.n_kv_heads + g) * 1000000 + pg);
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < m.n_q_heads; ++h) want[k(mk::OP_COMB)].insert((int64_t)b * m.n_q_heads + h);
    for (int r = 0; r < m.hidden; ++r) want[k(mk::OP_O)].insert(r), want[k(mk::OP_DOWN)].insert(r);
    if (moe) {
      for (int r = 0; r < m.n_experts; ++r) want[k(mk::OP_ROUTER)].insert(r);
      for (int b = 0; b < B; ++b)
        for (int j = 0; j < m.top_k; ++j)
          for (int f = 0; f < p->F; ++f) want[k(mk::OP_GATEUP)].insert(((int64_t)b * 64 + j) * 1000000 + f);
    } else {
      for (int f = 0; f < p->F; ++f) want[k(mk::OP_GATEUP)].insert(f);
    }
  }
  for (int r = 0; r < m.vocab; ++r) want[std::to_string(mk::OP_LM) + ":0"].insert(r);
  want[std::to_string(mk::OP_FINAL) + ":0"].insert(0);

  std::map<std::string, std::multiset<int64_t>> got;
  std::vector<uint32_t> producers(p->targets.size(), 0);
  std::vector<int> ctr_stage(p->targets.size(), -1);
  size_t k = 0;
  for (int cu = 0; cu < p->n_cu; ++cu) {
    int last = -1;
    for (auto& t : p->lists[cu]) {
      int st = p->stage_of_task[k++];
      if (st < last) return fail(MK_EINVAL, "validate: list of unit " + std::to_string(cu) + " is not in stage order");
      last = st;
      std::vector<std::pair<std::string, int64_t>> outs;
      task_outputs(p, t, outs);
      for (auto& [key, v] : outs) got[key].insert(v);
      if (t.signal != mk::NO_CTR) {
        if (t.signal >= p->targets.size()) return fail(MK_EINVAL, "validate: signal counter out of range");
        producers[t.signal]++;
        if (ctr_stage[t.signal] >= 0 && ctr_stage[t.signal] != st)
          return fail(MK_EINVAL, "validate: counter signalled from two stages");
        ctr_stage[t.signal] = st;
      }
    }
  }
  for (auto& [key, s] : want) {
    auto it = got.find(key);
    if (it == got.end()) return fail(MK_EINVAL, "validate: no task covers " + key);
    if (it->second.size() != s.size() || std::set<int64_t>(it->second.begin(), it->second.end()) != s)
      return fail(MK_EINVAL, "validate: outputs of " + key + " not covered exactly once");
  }
  if (got.size() != want.size()) return fail(MK_EINVAL, "validate: tasks of an unexpected kind");
  for (size_t c = 0; c < p->targets.size(); ++c)
    if (producers[c] != p->targets[c])
      return fail(MK_EINVAL, "validate: counter " + p->ctr_name[c] + " target != producer count");
  k = 0;
  for (int cu = 0; cu < p->n_cu; ++cu)
    for (auto& t : p->lists[cu]) {
      int st = p->stage_of_task[k++];
      for (auto [w, cnt] : {std::pair<uint16_t, uint16_t>{t.wait_a, t.cnt_a}, {t.wait_b, t.cnt_b}}) {
        if (w == mk::NO_CTR) continue;
        if (w >= p->targets.size()) return fail(MK_EINVAL, "validate: wait counter out of range");
        if (cnt != p->targets[w]) return fail(MK_EINVAL, "validate: wait count != target of " + p->ctr_name[w]);
        if (ctr_stage[w] >= st) return fail(MK_EINVAL, "validate: task waits on a counter of its own or a later stage");
      }
    }
  return MK_OK;
}

// ------------------------------------------------------------------ simulation

extern "C" mk_status mk_plan_simulate(const mk_plan_t* p, uint64_t seed, int32_t n_runs) {
  if (!p || n_runs <= 0) return fail(MK_EINVAL, "mk_plan_simulate: bad args");
  const auto& m = p->m;
  const int L = m.n_layers, Hkv = m.n_kv_heads, HG = p->HG;
  const bool moe = m.n_experts > 0;
  std::mt19937_64 rng(seed);
  std::vector<uint64_t> ctr(p->targets.size(), 0);
  // per-epoch completion counts by (op, layer, group) for the data-readiness check
  auto slot = [&](int op, int l, int g) { return ((size_t)op * (L + 1) + l) * (Hkv + 1) + g; };
  std::vector<uint32_t> total((mk::OP_COUNT + 1) * (L + 1) * (Hkv + 1), 0);
  for (int cu = 0; cu < p->n_cu; ++cu)
    for (auto& t : p->lists[cu]) {
      total[slot(t.op, t.layer, Hkv)]++;
      if (t.op == mk::OP_QKV || t.op == mk::OP_ATTN) total[slot(t.op, t.layer, t.op == mk::OP_QKV ? t.a0 : t.a1)]++;
    }
  for (int run = 0; run < n_runs; ++run) {
    const uint64_t epoch = (uint64_t)run + 1;
    std::vector<uint32_t> done(total.size(), 0);
    std::vector<size_t> head(p->n_cu, 0);
    auto all_done = [&](int op, int l, int g) { return done[slot(op, l, g)] == total[slot(op, l, g)]; };
    auto ready = [&](const Task& t) {
      if (t.wait_a != mk::NO_CTR && ctr[t.wait_a] < epoch * t.cnt_a) return false;
      if (t.wait_b != mk::NO_CTR && ctr[t.wait_b] < epoch * t.cnt_b) return false;
      return true;
    };
    // what each task reads must be complete when it runs (independent of the counters)
    auto inputs_ok = [&](const Task& t) -> bool {
      int l = t.layer;
      switch (t.op) {
        case mk::OP_QKV: return l == 0 || all_done(mk::OP_DOWN, l - 1, Hkv);
        case mk::OP_ATTN: return all_done(mk::OP_QKV, l, t.a1);
        case mk::OP_COMB: return all_done(mk::OP_ATTN, l, t.a1 / HG);
        case mk::OP_O: return all_done(mk::OP_COMB, l, Hkv);
        case mk::OP_ROUTER: return all_done(mk::OP_O, l, Hkv);
        case mk::OP_GATEUP: return all_done(mk::OP_O, l, Hkv) && (!moe || all_done(mk::OP_ROUTER, l, Hkv));
        case mk::OP_DOWN: return all_done(mk::OP_GATEUP, l, Hkv) && all_done(mk::OP_O, l, Hkv);
        case mk::OP_LM: return all_done(mk::OP_DOWN, L - 1, Hkv);
        case mk::OP_FINAL: return all_done(mk::OP_LM, 0, Hkv);
      }
      return false;
    };
    size_t remaining = p->n_tasks;
    std::vector<int> runnable;
    while (remaining) {
      runnable.clear();
      for (int cu = 0; cu < p->n_cu; ++cu)
        if (head[cu] < p->lists[cu].size() && ready(p->lists[cu][head[cu]])) runnable.push_back(cu);
      if (runnable.empty()) {
        std::string msg = "simulate: deadlock in epoch " + std::to_string(epoch) + "; blocked:";
        int shown = 0;
        for (int cu = 0; cu < p->n_cu && shown < 8; ++cu)
          if (head[cu] < p->lists[cu].size()) {
            const Task& t = p->lists[cu][head[cu]];
            msg += " unit " + std::to_string(cu) + " op " + std::to_string(t.op) + " layer " +
                   std::to_string(t.layer) + " waits " +
                   (t.wait_b != mk::NO_CTR ? p->ctr_name[t.wait_b] : std::string("-"));
            ++shown;
          }
        return fail(MK_ESTATE, msg);
      }
      // run a random prefix of runnable units, one task each, in random order
      std::shuffle(runnable.begin(), runnable.end(), rng);
      size_t n = 1 + rng() % runnable.size();
      for (size_t i = 0; i < n; ++i) {
        int cu = runnable[i];
        const Task& t = p->lists[cu][head[cu]];
        if (!inputs_ok(t))
          return fail(MK_ESTATE, "simulate: op " + std::to_string(t.op) + " layer " +
                                     std::to_string(t.layer) + " ran before its producers finished");
        head[cu]++;
        remaining--;
        done[slot(t.op, t.layer, Hkv)]++;
        if (t.op == mk::OP_QKV) done[slot(t.op, t.layer, t.a0)]++;
        if (t.op == mk::OP_ATTN) done[slot(t.op, t.layer, t.a1)]++;
        if (t.signal != mk::NO_CTR) ctr[t.signal]++;
      }
    }
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
  return p ? p->targets.size() * mk::CTR_STRIDE * 4 : 0;
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
  if (!p || !off || !bytes || which < 0 || which > 7) return fail(MK_EINVAL, "mk_plan_buffer: bad args");
  if (which < 7 && (layer < 0 || layer >= p->m.n_layers)) return fail(MK_EINVAL, "mk_plan_buffer: bad layer");
  *off = p->ws_off[which] + (which < 7 ? (size_t)layer * p->ws_stride[which] : 0);
  *bytes = p->ws_layer_bytes[which];
  return MK_OK;
}

extern "C" mk_status mk_plan_counter_targets(const mk_plan_t* p, uint32_t* out, int32_t n) {
  if (!p || !out || n < (int32_t)p->targets.size()) return fail(MK_EINVAL, "mk_plan_counter_targets: bad args");
  std::copy(p->targets.begin(), p->targets.end(), out);
  return MK_OK;
}

extern "C" void mk_plan_free(mk_plan_t* p) { delete p; }
