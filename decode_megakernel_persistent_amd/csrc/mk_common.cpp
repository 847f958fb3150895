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

// Pages, sequence slots and prefix checkpoints (kern page, "The runtime": a
// request leases its worst case and a slot, all or nothing; when it ends its
// pages freeze in place as a checkpoint; a later request with the same
// prefix shares the whole pages and gets a copy of the page the prefix ends
// inside; a token radix tree finds the longest checkpoint).
//
// ref[page] counts the page's holders: every live sequence whose list holds
// it, plus one while a checkpoint node holds it; a page is on the free list
// exactly when its count is zero. Checkpoint nodes form a tree with one page
// per node: a node's tokens are the tokens whose K/V its page holds (page_tokens
// of them, or fewer for the tail page of a sequence, which is always a leaf).
// Siblings never hold equal token runs.
struct mk_pool {
  struct Node {
    int32_t page = -1;  // -1: the root
    std::vector<int32_t> tokens;
    int32_t parent = -1;
    std::vector<int32_t> children;
    uint64_t tick = 0, order = 0;  // last use; insertion number
    bool alive = true;
  };
  int32_t n_pages, pt, n_slots;
  std::deque<int32_t> free_list;
  std::vector<char> slot_used;
  std::vector<int32_t> ref;
  std::vector<int32_t> node_of;  // checkpoint node holding a page, or -1
  std::map<int64_t, std::vector<int32_t>> pages;
  std::map<int64_t, int32_t> slot;
  std::vector<Node> nodes;  // nodes[0] is the root; a child's index exceeds its parent's
  uint64_t clock = 0, inserted = 0;
  int32_t cached = 0;  // live checkpoint nodes (= pages they hold)
};

extern "C" mk_status mk_pool_create(int32_t n_pages, int32_t pt, int32_t n_slots,
                                    const int32_t* order, mk_pool_t** out) {
  if (!out || n_pages < 0 || pt <= 0 || n_slots <= 0) return fail(MK_EINVAL, "mk_pool_create: bad args");
  auto* p = new mk_pool();
  p->n_pages = n_pages;
  p->pt = pt;
  p->n_slots = n_slots;
  p->slot_used.assign(n_slots, 0);
  p->ref.assign(n_pages, 0);
  p->node_of.assign(n_pages, -1);
  p->nodes.emplace_back();
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

namespace {

int32_t pages_for(const mk_pool* p, int64_t tokens) { return (int32_t)((tokens + p->pt - 1) / p->pt); }

int32_t lowest_free_slot(const mk_pool* p) {
  for (int32_t i = 0; i < p->n_slots; ++i)
    if (!p->slot_used[i]) return i;
  return -1;
}

// Checkpoint pages that evictions could free: the nodes of every subtree in
// which no page has a holder besides its node (children before parents).
int64_t evictable(const mk_pool* p) {
  std::vector<char> ev(p->nodes.size(), 0);
  int64_t n = 0;
  for (size_t i = p->nodes.size(); i-- > 1;) {
    const auto& nd = p->nodes[i];
    if (!nd.alive || p->ref[nd.page] != 1) continue;
    bool all = true;
    for (int32_t c : nd.children) all = all && ev[c];
    if (all) {
      ev[i] = 1;
      ++n;
    }
  }
  return n;
}

// Evict the least recently used leaf whose page only its node holds (ties:
// the earlier inserted); its page goes to the back of the free list.
bool evict_one(mk_pool* p) {
  int32_t best = -1;
  for (size_t i = 1; i < p->nodes.size(); ++i) {
    const auto& nd = p->nodes[i];
    if (!nd.alive || !nd.children.empty() || p->ref[nd.page] != 1) continue;
    if (best < 0 || nd.tick < p->nodes[best].tick ||
        (nd.tick == p->nodes[best].tick && nd.order < p->nodes[best].order))
      best = (int32_t)i;
  }
  if (best < 0) return false;
  auto& nd = p->nodes[best];
  nd.alive = false;
  auto& sib = p->nodes[nd.parent].children;
  sib.erase(std::find(sib.begin(), sib.end(), best));
  p->ref[nd.page] = 0;
  p->node_of[nd.page] = -1;
  p->free_list.push_back(nd.page);
  --p->cached;
  return true;
}

// Make n pages free, evicting checkpoints under pressure; all or nothing.
bool ensure_free(mk_pool* p, int64_t n) {
  if ((int64_t)p->free_list.size() >= n) return true;
  if ((int64_t)p->free_list.size() + evictable(p) < n) return false;
  while ((int64_t)p->free_list.size() < n) evict_one(p);
  return true;
}

std::vector<int32_t> take_free(mk_pool* p, int32_t n) {
  std::vector<int32_t> got(p->free_list.begin(), p->free_list.begin() + n);
  p->free_list.erase(p->free_list.begin(), p->free_list.begin() + n);
  for (int32_t pg : got) p->ref[pg] = 1;
  return got;
}

// Longest checkpointed prefix of tokens[0, limit): the full nodes matched
// whole (path) and the node the match ends inside (-1: none). At each page
// the child with the longest common run wins (ties: the earlier inserted).
int32_t match_prefix(const mk_pool* p, const int32_t* tokens, int32_t limit, std::vector<int32_t>& path,
                     int32_t* inside) {
  int32_t node = 0, pos = 0;
  *inside = -1;
  while (pos < limit) {
    const int32_t span = std::min(p->pt, limit - pos);
    int32_t best = -1, best_n = 0;
    for (int32_t c : p->nodes[node].children) {
      const auto& t = p->nodes[c].tokens;
      int32_t n = 0;
      while (n < span && n < (int32_t)t.size() && t[n] == tokens[pos + n]) ++n;
      if (n > best_n || (n == best_n && n > 0 && p->nodes[c].order < p->nodes[best].order)) {
        best = c;
        best_n = n;
      }
    }
    if (best < 0) break;
    if (best_n == p->pt) {
      path.push_back(best);
      node = best;
      pos += p->pt;
      continue;
    }
    *inside = best;
    pos += best_n;
    break;
  }
  return pos;
}

mk_status lease_impl(mk_pool* p, int64_t seq, const int32_t* prompt, int32_t n_prompt, int32_t tokens,
                     int32_t* slot_out, int32_t* matched, int32_t* copy_src, int32_t* copy_dst,
                     const char* who) {
  if (p->pages.count(seq)) return fail(MK_ESTATE, std::string(who) + ": sequence already holds a lease");
  const int32_t slot = lowest_free_slot(p);
  if (slot < 0) return fail(MK_ENOMEM, std::string(who) + ": no free sequence slot");
  std::vector<int32_t> path;
  int32_t inside = -1, m = 0;
  // the prompt's last token always runs: it gives the next token's logits
  if (prompt && n_prompt > 1) m = match_prefix(p, prompt, n_prompt - 1, path, &inside);
  const int32_t need = pages_for(p, tokens) - (int32_t)path.size();
  // pin what the lease reuses, so that no eviction takes it
  for (int32_t n : path) ++p->ref[p->nodes[n].page];
  if (inside >= 0) ++p->ref[p->nodes[inside].page];
  if (!ensure_free(p, need)) {
    for (int32_t n : path) --p->ref[p->nodes[n].page];
    if (inside >= 0) --p->ref[p->nodes[inside].page];
    return fail(MK_ENOMEM, std::string(who) + ": " + std::to_string(need) + " pages needed, " +
                               std::to_string(p->free_list.size()) + " free and " +
                               std::to_string(evictable(p)) + " held by checkpoints no one reads");
  }
  std::vector<int32_t> list;
  for (int32_t n : path) {
    list.push_back(p->nodes[n].page);
    p->nodes[n].tick = ++p->clock;
  }
  const std::vector<int32_t> fresh = take_free(p, need);
  list.insert(list.end(), fresh.begin(), fresh.end());
  if (inside >= 0) {
    --p->ref[p->nodes[inside].page];
    p->nodes[inside].tick = ++p->clock;
  }
  p->pages[seq] = std::move(list);
  p->slot_used[slot] = 1;
  p->slot[seq] = slot;
  if (slot_out) *slot_out = slot;
  if (matched) *matched = m;
  if (copy_src) *copy_src = inside >= 0 ? p->nodes[inside].page : -1;
  if (copy_dst) *copy_dst = inside >= 0 ? fresh[0] : -1;
  return MK_OK;
}

}  // namespace

extern "C" mk_status mk_pool_lease(mk_pool_t* p, int64_t seq, int32_t tokens, int32_t* slot_out) {
  if (!p || tokens < 0) return fail(MK_EINVAL, "mk_pool_lease: bad args");
  return lease_impl(p, seq, nullptr, 0, tokens, slot_out, nullptr, nullptr, nullptr, "mk_pool_lease");
}

extern "C" mk_status mk_pool_lease_prefix(mk_pool_t* p, int64_t seq, const int32_t* prompt, int32_t n_prompt,
                                          int32_t tokens, int32_t* slot_out, int32_t* matched,
                                          int32_t* copy_src, int32_t* copy_dst) {
  if (!p || (!prompt && n_prompt) || n_prompt < 0 || tokens < n_prompt)
    return fail(MK_EINVAL, "mk_pool_lease_prefix: bad args (worst case below the prompt length?)");
  return lease_impl(p, seq, prompt, n_prompt, tokens, slot_out, matched, copy_src, copy_dst,
                    "mk_pool_lease_prefix");
}

extern "C" mk_status mk_pool_extend(mk_pool_t* p, int64_t seq, int32_t tokens) {
  if (!p) return fail(MK_EINVAL, "mk_pool_extend: bad args");
  auto it = p->pages.find(seq);
  if (it == p->pages.end()) return fail(MK_ESTATE, "mk_pool_extend: sequence not leased");
  int32_t need = pages_for(p, tokens) - (int32_t)it->second.size();
  if (need <= 0) return MK_OK;
  if (!ensure_free(p, need)) return fail(MK_ENOMEM, "mk_pool_extend: pool exhausted");
  const std::vector<int32_t> fresh = take_free(p, need);
  it->second.insert(it->second.end(), fresh.begin(), fresh.end());
  return MK_OK;
}

extern "C" mk_status mk_pool_release(mk_pool_t* p, int64_t seq) {
  if (!p) return fail(MK_EINVAL, "mk_pool_release: bad args");
  auto it = p->pages.find(seq);
  if (it == p->pages.end()) return fail(MK_ESTATE, "mk_pool_release: sequence not leased");
  for (int32_t pg : it->second)
    if (--p->ref[pg] == 0) p->free_list.push_back(pg);
  p->pages.erase(it);
  p->slot_used[p->slot[seq]] = 0;
  p->slot.erase(seq);
  return MK_OK;
}

extern "C" mk_status mk_pool_finish(mk_pool_t* p, int64_t seq, const int32_t* tokens, int32_t n_tokens) {
  if (!p || (!tokens && n_tokens) || n_tokens < 0) return fail(MK_EINVAL, "mk_pool_finish: bad args");
  auto it = p->pages.find(seq);
  if (it == p->pages.end()) return fail(MK_ESTATE, "mk_pool_finish: sequence not leased");
  const std::vector<int32_t>& list = it->second;
  if (pages_for(p, n_tokens) > (int32_t)list.size())
    return fail(MK_EBOUNDS, "mk_pool_finish: more tokens than the sequence's pages hold");
  // freeze the pages holding tokens 0 .. n_tokens-1 along the token path; a
  // run that the tree already holds keeps its node (this page is then freed).
  // Below the first run the tree lacks, every page becomes a new node, and
  // none of those may already be a checkpoint's (tokens that disagree with
  // a shared page's).
  auto run_at = [&](int32_t j) {
    const int32_t n = std::min(p->pt, n_tokens - j * p->pt);
    return std::vector<int32_t>(tokens + (size_t)j * p->pt, tokens + (size_t)j * p->pt + n);
  };
  auto child_with = [&](int32_t node, const std::vector<int32_t>& run) {
    for (int32_t c : p->nodes[node].children)
      if (p->nodes[c].tokens == run) return c;
    return -1;
  };
  {
    int32_t node = 0;
    for (int32_t j = 0; j * p->pt < n_tokens; ++j) {
      const int32_t hit = node >= 0 ? child_with(node, run_at(j)) : -1;
      if (hit < 0 && p->node_of[list[j]] >= 0)
        return fail(MK_EINVAL, "mk_pool_finish: the tokens of page " + std::to_string(j) +
                                   " disagree with the checkpoint the sequence shares there");
      node = hit;
    }
  }
  int32_t node = 0;
  for (int32_t j = 0; j * p->pt < n_tokens; ++j) {
    const std::vector<int32_t> run = run_at(j);
    int32_t hit = child_with(node, run);
    if (hit < 0) {
      mk_pool::Node nd;
      nd.page = list[j];
      nd.tokens = run;
      nd.parent = node;
      nd.order = ++p->inserted;
      p->nodes.push_back(std::move(nd));
      hit = (int32_t)p->nodes.size() - 1;
      p->nodes[node].children.push_back(hit);
      p->node_of[list[j]] = hit;
      ++p->ref[list[j]];
      ++p->cached;
    }
    p->nodes[hit].tick = ++p->clock;
    node = hit;
  }
  return mk_pool_release(p, seq);
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
extern "C" int32_t mk_pool_cached_pages(const mk_pool_t* p) { return p ? p->cached : -1; }
extern "C" int32_t mk_pool_seq_pages(const mk_pool_t* p, int64_t seq) {
  if (!p) return -1;
  auto it = p->pages.find(seq);
  return it == p->pages.end() ? -1 : (int32_t)it->second.size();
}
extern "C" void mk_pool_free(mk_pool_t* p) { delete p; }
