// Errors, model-level helpers (rotary tables, byte accounting), pool.
#include <cmath>
#include <cstring>
#include <deque>
#include <map>
#include <string>
#include <vector>
#include <algorithm>

#include "mk.h"
#include "mk_plan.hpp"

namespace mkh {
static thread_local std::string g_err;
void set_error(const std::string& s) { g_err = s; }
mk_status fail(mk_status st, const std::string& s) {
  g_err = s;
  return st;
}
}  // namespace mkh

using mkh::fail;

extern "C" int32_t mk_abi_version(void) { return MK_ABI_VERSION; }
extern "C" const char* mk_last_error(void) { return mkh::g_err.c_str(); }

// Rotary angle p * theta^(-2i/d) in fp64, cos and sin rounded to fp32.
extern "C" mk_status mk_rope_table(float theta, int32_t d, int32_t n_pos, float* c, float* s) {
  if (!c || !s || d <= 0 || (d & 1) || n_pos < 0) return fail(MK_EINVAL, "mk_rope_table: bad args");
  const int h = d / 2;
  std::vector<double> inv(h);
  for (int i = 0; i < h; ++i) inv[i] = std::pow((double)theta, -2.0 * i / d);
  for (int64_t p = 0; p < n_pos; ++p)
    for (int i = 0; i < h; ++i) {
      double a = (double)p * inv[i];
      c[p * h + i] = (float)std::cos(a);
      s[p * h + i] = (float)std::sin(a);
    }
  return MK_OK;
}

extern "C" int64_t mk_kv_pool_elems(const mk_model_desc* m, int64_t n_pages) {
  if (!m) return -1;
  return n_pages * (int64_t)m->n_layers * m->n_kv_heads * 2 * m->page_tokens * m->head_dim;
}

extern "C" mk_status mk_step_bytes(const mk_model_desc* m, int32_t batch, const int32_t* seq_lens,
                                   const int32_t* distinct, double* wb, double* kr, double* kw) {
  if (!m || !seq_lens || batch <= 0 || !wb || !kr || !kw) return fail(MK_EINVAL, "mk_step_bytes: bad args");
  const double L = m->n_layers, H = m->hidden, Hq = m->n_q_heads, Hkv = m->n_kv_heads,
               d = m->head_dim;
  double w = L * (H * (Hq + 2 * Hkv) * d + Hq * d * H);
  if (m->n_experts > 0) {
    w += L * H * m->n_experts;
    for (int l = 0; l < m->n_layers; ++l) {
      double de = distinct ? distinct[l] : std::min<double>(m->n_experts, (double)batch * m->top_k);
      w += de * 3.0 * H * m->expert_ffn;
    }
  } else {
    w += L * 3.0 * H * m->ffn_dim;
  }
  w += (double)m->vocab * H + batch * H + (2 * L + 1) * H;
  const double per_tok = L * 2 * Hkv * d * 2;
  double r = 0;
  for (int b = 0; b < batch; ++b) r += ((double)seq_lens[b] + 1) * per_tok;
  *wb = 2 * w;
  *kr = r;
  *kw = batch * per_tok;
  return MK_OK;
}

// ------------------------------------------------------------------ pool

struct mk_pool {
  int32_t n_pages, pt, n_slots;
  std::deque<int32_t> free_list;
  std::vector<char> slot_used;
  std::map<int64_t, std::vector<int32_t>> pages;
  std::map<int64_t, int32_t> slot;
};

extern "C" mk_status mk_pool_create(int32_t n_pages, int32_t pt, int32_t n_slots,
                                    const int32_t* order, mk_pool_t** out) {
  if (!out || n_pages < 0 || pt <= 0 || n_slots <= 0) return fail(MK_EINVAL, "mk_pool_create: bad args");
  auto* p = new mk_pool();
  p->n_pages = n_pages;
  p->pt = pt;
  p->n_slots = n_slots;
  p->slot_used.assign(n_slots, 0);
  std::vector<char> seen(n_pages, 0);
  for (int32_t i = 0; i < n_pages; ++i) {
    int32_t v = order ? order[i] : i;
    if (v < 0 || v >= n_pages || seen[v]) {
      delete p;
      return fail(MK_EINVAL, "mk_pool_create: initial_order is not a permutation of [0, n_pages)");
    }
    seen[v] = 1;
    p->free_list.push_back(v);
  }
  *out = p;
  return MK_OK;
}

static int32_t pages_for(const mk_pool* p, int64_t tokens) {
  return (int32_t)((tokens + p->pt - 1) / p->pt);
}

extern "C" mk_status mk_pool_lease(mk_pool_t* p, int64_t seq, int32_t tokens, int32_t* slot_out) {
  if (!p || tokens < 0) return fail(MK_EINVAL, "mk_pool_lease: bad args");
  if (p->pages.count(seq)) return fail(MK_ESTATE, "mk_pool_lease: sequence already holds a lease");
  int32_t need = pages_for(p, tokens);
  int32_t slot = -1;
  for (int32_t i = 0; i < p->n_slots; ++i)
    if (!p->slot_used[i]) { slot = i; break; }
  if (slot < 0) return fail(MK_ENOMEM, "mk_pool_lease: no free sequence slot");
  if (need > (int32_t)p->free_list.size())
    return fail(MK_ENOMEM, "mk_pool_lease: " + std::to_string(need) + " pages needed, " +
                               std::to_string(p->free_list.size()) + " free");
  std::vector<int32_t> got(p->free_list.begin(), p->free_list.begin() + need);
  p->free_list.erase(p->free_list.begin(), p->free_list.begin() + need);
  p->pages[seq] = std::move(got);
  p->slot_used[slot] = 1;
  p->slot[seq] = slot;
  if (slot_out) *slot_out = slot;
  return MK_OK;
}

extern "C" mk_status mk_pool_extend(mk_pool_t* p, int64_t seq, int32_t tokens) {
  if (!p) return fail(MK_EINVAL, "mk_pool_extend: bad args");
  auto it = p->pages.find(seq);
  if (it == p->pages.end()) return fail(MK_ESTATE, "mk_pool_extend: sequence not leased");
  int32_t need = pages_for(p, tokens) - (int32_t)it->second.size();
  if (need <= 0) return MK_OK;
  if (need > (int32_t)p->free_list.size()) return fail(MK_ENOMEM, "mk_pool_extend: pool exhausted");
  for (int32_t i = 0; i < need; ++i) {
    it->second.push_back(p->free_list.front());
    p->free_list.pop_front();
  }
  return MK_OK;
}

extern "C" mk_status mk_pool_release(mk_pool_t* p, int64_t seq) {
  if (!p) return fail(MK_EINVAL, "mk_pool_release: bad args");
  auto it = p->pages.find(seq);
  if (it == p->pages.end()) return fail(MK_ESTATE, "mk_pool_release: sequence not leased");
  for (int32_t pg : it->second) p->free_list.push_back(pg);
  p->pages.erase(it);
  p->slot_used[p->slot[seq]] = 0;
  p->slot.erase(seq);
  return MK_OK;
}

extern "C" mk_status mk_pool_page_table(const mk_pool_t* p, const int64_t* ids, int32_t n,
                                        int32_t max_pages, int32_t* out) {
  if (!p || (!ids && n) || !out || max_pages < 0) return fail(MK_EINVAL, "mk_pool_page_table: bad args");
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->pages.find(ids[i]);
    if (it == p->pages.end()) return fail(MK_ESTATE, "mk_pool_page_table: sequence not leased");
    if ((int32_t)it->second.size() > max_pages)
      return fail(MK_EBOUNDS, "mk_pool_page_table: sequence holds more pages than max_pages");
    for (int32_t j = 0; j < max_pages; ++j)
      out[(int64_t)i * max_pages + j] = j < (int32_t)it->second.size() ? it->second[j] : -1;
  }
  return MK_OK;
}

extern "C" int32_t mk_pool_free_pages(const mk_pool_t* p) { return p ? (int32_t)p->free_list.size() : -1; }
extern "C" int32_t mk_pool_seq_pages(const mk_pool_t* p, int64_t seq) {
  if (!p) return -1;
  auto it = p->pages.find(seq);
  return it == p->pages.end() ? -1 : (int32_t)it->second.size();
}
extern "C" void mk_pool_free(mk_pool_t* p) { delete p; }
