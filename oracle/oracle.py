"""CPU oracle of one decode step over a paged KV cache.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in oracle/. The
product path (the HIP library and its binding) never does, and shares no
code with it: the only common module is fixtures/, which draws the seeded
inputs and holds none of the step's arithmetic.

What it computes. The megakernel page ("Inside the megakernel serving
engine for North Mini Code", introduction) states that the megakernel is
ordinary tiled GEMMs and ordinary paged attention restructured into one
persistent kernel; section "What is a Megakernel?" states that it runs the
entire forward pass. The step is therefore the plain decoder step, written
here op by op in the order the step takes them, per sequence (batch rows
are independent; the Kinetic book, "Adding a weight format or a kernel",
requires each batch row to equal the single-row result):

  x = E[token]
  per layer: u = rmsnorm(x); q,k,v = W_qkv u; rotate q,k at position p;
             append bf16(k), bf16(v); o = softmax(q K^T / sqrt(d)) V per
             query head (grouped-query); x += W_o o; u = rmsnorm(x);
             dense:  x += W_down (silu(W_gate u) * W_up u)
             MoE:    pi = softmax(W_r u); top-k of pi; renormalised weights;
                     x += sum_j w_j W_down,j (silu(W_gate,j u) * W_up,j u)
  z = rmsnorm(x); logits = W_lm z; next = argmax(logits)

Readings where the pages are silent (each listed in the design notes):
RMSNorm gains are 1.0; rotary uses the half-split ("NeoX") layout with
theta_i = theta^(-2i/d) and cos/sin computed in fp64, rounded to fp32;
the new token sits at position p = number of cached tokens and attends to
itself through its bf16-rounded k and v; score scale 1/sqrt(d); GQA maps
query head h to kv head h // (Hq/Hkv); the router takes a softmax over all
experts, keeps the top k (ties to the lower index) and renormalises over
them; argmax ties go to the lower index; the LM head is untied.

Precision. The decode step is specified as fp32 math on bf16 weights: `dt` defaults
to torch.float32; torch.float64 is a cross-check mode. Weights are the
same bf16 bits as the GPU's, widened exactly. Decisions (top-k, argmax)
are taken in the working precision.

Library primitives used as steps: matrix-vector products (torch.mv), the
stable sort (torch.sort(stable=True)) and torch.argmax (first maximum).
"""
import copy
import math
from collections import deque

import torch


# ---------------------------------------------------------------- elementary ops

def widen(w, dt):
    """bf16 tensor -> working precision (exact)."""
    return w.to(dt)


def to_bf16(x):
    """Round to bf16, nearest-even, through fp32 (the storage precision of KV)."""
    return x.to(torch.float32).to(torch.bfloat16)


def rmsnorm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g."""
    dt = x.dtype
    return x / torch.sqrt((x * x).mean() + eps) * widen(g, dt)


def matvec(w, u):
    """y = W u for W bf16 [rows][cols] (row-major [out][in])."""
    return torch.mv(widen(w, u.dtype), u)


def rope_cos_sin(theta, d, pos):
    """cos/sin of pos * theta^(-2i/d), i < d/2, in fp64, rounded to fp32."""
    i = torch.arange(d // 2, dtype=torch.float64)
    ang = float(pos) * torch.pow(torch.tensor(float(theta), dtype=torch.float64), -2.0 * i / d)
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def rope(v, cos, sin):
    """Rotate rows of v [n][d] by pairs (i, i + d/2): (a, b) -> (a c - b s, b c + a s)."""
    d = v.shape[-1]
    c, s = cos.to(v.dtype), sin.to(v.dtype)
    a, b = v[..., : d // 2], v[..., d // 2:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def softmax(s):
    """exp(s - max s) / sum exp(s - max s) along the last axis."""
    e = torch.exp(s - s.max(dim=-1, keepdim=True).values)
    return e / e.sum(dim=-1, keepdim=True)


def attention(q, K, V):
    """Plain softmax attention of queries q [n][d] over K, V [T][d] (bf16 or float)."""
    dt = q.dtype
    d = q.shape[-1]
    s = (q @ widen(K, dt).T) / math.sqrt(d)
    return softmax(s) @ widen(V, dt)


def gather_pages(pool, page_row, n_tok, pt):
    """Contiguous [n_tok][d] view of a paged store pool [n_pages][pt][d] through page_row."""
    n_pg = (n_tok + pt - 1) // pt
    rows = [pool[int(page_row[j])] for j in range(n_pg)]
    return torch.cat(rows, dim=0)[:n_tok]


def attention_paged(q, pool_k, pool_v, page_row, n_tok, pt):
    """Paged attention: gather K, V through the page table, then attend."""
    return attention(q, gather_pages(pool_k, page_row, n_tok, pt),
                     gather_pages(pool_v, page_row, n_tok, pt))


def attention_partial(q, K, V):
    """Unnormalised partial over one key range: (o = sum_j e^{s_j - m} v_j, m, l)."""
    dt = q.dtype
    d = q.shape[-1]
    s = (q @ widen(K, dt).T) / math.sqrt(d)
    m = s.max(dim=-1).values
    e = torch.exp(s - m[:, None])
    return e @ widen(V, dt), m, e.sum(dim=-1)


def merge_partials(parts):
    """Log-sum-exp merge of partials (o, m, l) over disjoint key ranges, in list order."""
    M = torch.stack([m for _, m, _ in parts]).max(dim=0).values
    o = torch.zeros_like(parts[0][0])
    L = torch.zeros_like(parts[0][1])
    for oi, mi, li in parts:
        c = torch.exp(mi - M)
        o = o + c[:, None] * oi
        L = L + c * li
    return o / L[:, None]


def topk(p, k):
    """Indices of the k largest entries, descending, ties to the lower index."""
    _, idx = torch.sort(-p, stable=True)
    return idx[:k]


def route(r, k, norm_topk=True):
    """pi = softmax(r); ids = top-k of pi; w = pi[ids] (/ sum pi[ids] if norm_topk)."""
    pi = softmax(r)
    ids = topk(pi, k)
    w = pi[ids]
    if norm_topk:
        w = w / w.sum()
    return ids, w


def route_given(r, ids, norm_topk=True):
    """Routing weights of a given selection: w = pi[ids] (/ sum pi[ids])."""
    pi = softmax(r)
    ids = torch.as_tensor(list(ids), dtype=torch.int64)
    w = pi[ids]
    if norm_topk:
        w = w / w.sum()
    return ids, w


def silu(z):
    return z / (1.0 + torch.exp(-z))


def swiglu(wg, wu, u):
    """silu(W_gate u) * (W_up u)."""
    return silu(matvec(wg, u)) * matvec(wu, u)


def argmax(v):
    """Index of the largest entry, ties to the lower index."""
    return int(torch.argmax(v))


# ---------------------------------------------------------------- KV state

def prefill(m, W, kv, tokens, dt=torch.float32):
    """A prompt chunk of one sequence (batch row 0 of kv): the decode step of
    each token in order, each attending to every token before it. A prefill
    computes the same K, V and hidden states as decoding the prompt one token
    at a time; this is that definition (the megakernel page's continuous
    batching fills pages from prompts; the pages give no separate prefill
    arithmetic). Returns the list of per-token step results."""
    return [decode_step(m, W, kv, [t], dt) for t in tokens]


def sample_next(logits, temperature, top_k, top_p, min_p, u, k_max=64):
    """The next token drawn from one sequence's logits, in fp64.

    The Kinetic book ("Pick the sampling", the sampler flags) runs the
    llama.cpp samplers in their default order; of them this takes top-k,
    top-p, min-p and temperature, in that order, then one draw, and
    temperature 0 always takes the likeliest token. Readings: ties in the
    logits rank the lower id first; top_k outside 1 .. k_max means k_max (the
    device keeps at most k_max candidates); top-p keeps the shortest run of
    candidates, most likely first, whose probabilities (softmax over the
    candidates at temperature 1) sum to at least top_p; min-p keeps the
    candidates at least min_p times as likely as the best; the best
    candidate is always kept; the draw takes the first kept candidate, most
    likely first, at which the running sum of exp((z - z_max) / T) exceeds
    u times its total (u in [0, 1) is given, not drawn here).
    """
    z = logits.double()
    if temperature <= 0:
        return argmax(z)
    k = top_k if 1 <= top_k <= k_max else k_max
    k = min(k, z.numel())
    if k == 1:
        return argmax(z)
    _, order = torch.sort(-z, stable=True)       # descending, equal values by lower id
    cand = order[:k]
    zc = z[cand]
    p = torch.softmax(zc, dim=0)
    keep = torch.ones(k, dtype=torch.bool)
    if top_p < 1:
        cum = torch.cumsum(p, dim=0)
        reach = int(torch.nonzero(cum >= top_p)[0]) if bool((cum >= top_p).any()) else k - 1
        keep[reach + 1:] = False
    if min_p > 0:
        keep &= p >= min_p * p[0]
    keep[0] = True
    w = torch.where(keep, torch.exp((zc - zc[0]) / temperature), torch.zeros_like(zc))
    run = torch.cumsum(w, dim=0)
    hit = torch.nonzero(keep & (run > u * run[-1]))
    pick = int(hit[0]) if hit.numel() else int(torch.nonzero(keep)[-1])
    return int(cand[pick])


class OracleKV:
    """Contiguous bf16 KV per (layer, sequence, kv head), with a length per sequence."""

    def __init__(self, m, ctx, cap_extra, kv_src=None):
        L, Hkv, d = m["n_layers"], m["n_kv_heads"], m["head_dim"]
        self.m = m
        self.len = list(ctx)
        self.K, self.V = {}, {}
        for b, c in enumerate(ctx):
            cap = c + cap_extra
            for l in range(L):
                for g in range(Hkv):
                    K = torch.zeros(cap, d, dtype=torch.bfloat16)
                    V = torch.zeros(cap, d, dtype=torch.bfloat16)
                    if kv_src is not None and c > 0:
                        K[:c] = kv_src.k(l, b, g, c)
                        V[:c] = kv_src.v(l, b, g, c)
                    self.K[l, b, g] = K
                    self.V[l, b, g] = V

    def append(self, l, b, g, k, v):
        p = self.len[b]
        self.K[l, b, g][p] = k
        self.V[l, b, g][p] = v

    def keys(self, l, b, g, n):
        return self.K[l, b, g][:n]

    def values(self, l, b, g, n):
        return self.V[l, b, g][:n]


# ---------------------------------------------------------------- the step

def decode_step(m, W, kv, tokens, dt=torch.float32, force_ids=None):
    """One decode step for every sequence b: token tokens[b] at position kv.len[b].

    Returns a dict with per-sequence lists: next (int), logits [V],
    x_attn[l] / x_ffn[l] (hidden after each residual), topk_ids[l],
    topk_w[l], router_logits[l], k_new[l] / v_new[l] (bf16 [Hkv][d]).
    The KV state gains one token per sequence.

    force_ids: optional {(b, l): k expert ids}. Where the router's k-th and
    (k+1)-th probabilities tie to within fp32 rounding, two correct
    implementations may select different experts; a comparison then
    continues from the other side's selection: the listed ids replace the
    top-k of sequence b at layer l, and their weights are the same
    probabilities of the same softmax, renormalised over those ids.
    """
    L, H, Hq, Hkv, d = m["n_layers"], m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    hg = Hq // Hkv
    eps = m["rms_eps"]
    moe = m["n_experts"] > 0
    out = {k: [] for k in ("next", "logits", "x_attn", "x_ffn", "topk_ids", "topk_w",
                           "router_logits", "k_new", "v_new")}
    for b, tok in enumerate(tokens):
        pos = kv.len[b]
        cos, sin = rope_cos_sin(m["rope_theta"], d, pos)
        x = widen(W.embed_row(int(tok)), dt)
        xa, xf, ids_l, w_l, r_l, kn_l, vn_l = [], [], [], [], [], [], []
        for l in range(L):
            u = rmsnorm(x, W.attn_norm(l), eps)
            qkv = matvec(W.wqkv(l), u)
            q = rope(qkv[: Hq * d].view(Hq, d), cos, sin)
            k = rope(qkv[Hq * d: (Hq + Hkv) * d].view(Hkv, d), cos, sin)
            v = qkv[(Hq + Hkv) * d:].view(Hkv, d)
            kb, vb = to_bf16(k), to_bf16(v)
            for g in range(Hkv):
                kv.append(l, b, g, kb[g], vb[g])
            kn_l.append(kb)
            vn_l.append(vb)
            o = torch.empty(Hq, d, dtype=dt)
            for g in range(Hkv):
                o[g * hg:(g + 1) * hg] = attention(q[g * hg:(g + 1) * hg],
                                                   kv.keys(l, b, g, pos + 1),
                                                   kv.values(l, b, g, pos + 1))
            x = x + matvec(W.wo(l), o.reshape(-1))
            xa.append(x.clone())
            u = rmsnorm(x, W.ffn_norm(l), eps)
            if moe:
                r = matvec(W.router(l), u)
                if force_ids is not None and (b, l) in force_ids:
                    ids, wts = route_given(r, force_ids[b, l], bool(m["norm_topk"]))
                else:
                    ids, wts = route(r, m["top_k"], bool(m["norm_topk"]))
                y = torch.zeros(H, dtype=dt)
                for j in range(m["top_k"]):
                    e = int(ids[j])
                    y = y + wts[j] * matvec(W.down(l, e), swiglu(W.gate(l, e), W.up(l, e), u))
                x = x + y
                ids_l.append(ids.clone())
                w_l.append(wts.clone())
                r_l.append(r.clone())
            else:
                x = x + matvec(W.down(l), swiglu(W.gate(l), W.up(l), u))
            xf.append(x.clone())
        z = rmsnorm(x, W.final_norm(), eps)
        logits = matvec(W.lm_head(), z)
        out["next"].append(argmax(logits))
        out["logits"].append(logits)
        out["x_attn"].append(xa)
        out["x_ffn"].append(xf)
        out["topk_ids"].append(ids_l)
        out["topk_w"].append(w_l)
        out["router_logits"].append(r_l)
        out["k_new"].append(kn_l)
        out["v_new"].append(vn_l)
    for b in range(len(tokens)):
        kv.len[b] += 1
    return out


def near_tie(r, k, rel):
    """True when the k-th and (k+1)-th largest softmax probabilities of the
    router logits r differ by less than rel of the k-th: fp32 logits summed
    in another order can then rank them either way."""
    p = softmax(r.double())
    s = torch.sort(p, descending=True).values
    return k < s.numel() and (s[k - 1] - s[k]).item() < rel * s[k - 1].item()


def ids_near_tie(r, mine, theirs, rel):
    """True when the id lists mine and theirs can both be the descending
    ranking of the softmax probabilities of router logits r, up to rounding:
    at every slot where they differ, the two experts' probabilities differ by
    less than rel of the larger. This covers a different k-th expert (the
    k-th and (k+1)-th nearly tie, as near_tie) and two selected experts in
    the other order (slot order is the ranking, and fp32 logits summed in
    another order can rank nearly equal probabilities either way)."""
    p = softmax(r.double())
    for a, b in zip(mine, theirs):
        if a != b:
            pa, pb = p[int(a)].item(), p[int(b)].item()
            if abs(pa - pb) >= rel * max(pa, pb):
                return False
    return True


def decode_step_following(m, W, kv, tokens, other_ids, rel, dt=torch.float32):
    """decode_step, continuing from another implementation's routing where
    the two may both be right.

    other_ids[b][l]: the other side's k expert ids of sequence b at layer l.
    Where the oracle's own top-k differs from them and the two lists are a
    near-tie (ids_near_tie(router logits, mine, theirs, rel)), the other side's ids are
    taken at that layer (force_ids of decode_step) and the step is run again
    from the start, so that later layers are compared on the same routing.
    Returns (out, forced, differ): forced lists the (b, l) taken from
    other_ids; differ lists the (b, l) where the ids differ without a
    near-tie. The KV state gains one token per sequence, as in decode_step.
    """
    start = list(kv.len)
    force = {}
    k = m["top_k"]
    while True:
        kv.len = list(start)
        out = decode_step(m, W, kv, tokens, dt, force_ids=force)
        if not m["n_experts"]:
            return out, [], []
        new, differ = None, []
        for b in range(len(tokens)):
            for l in range(m["n_layers"]):
                mine = [int(v) for v in out["topk_ids"][b][l]]
                theirs = [int(v) for v in other_ids[b][l]]
                if mine == theirs or (b, l) in force:
                    continue
                if ids_near_tie(out["router_logits"][b][l], mine, theirs, rel):
                    new = (b, l, theirs)
                    break
                differ.append((b, l))
                break  # later layers of this sequence follow another routing
            if new:
                break
        if new is None:
            return out, sorted(force), differ
        force[new[0], new[1]] = new[2]


# ---------------------------------------------------------------- speed-of-light

def step_bytes(m, ctx, distinct_experts=None):
    """Algorithmic HBM bytes of one step: (weights, kv_read, kv_write).

    Weights read once per step: per layer W_qkv, W_o, router and the experts
    actually selected (distinct per layer, all batch rows together), plus the
    LM head, one embedding row per sequence and the norm gains. KV: every
    cached token of every layer and kv head is read (including the new one),
    and the new token's K and V are written.
    """
    L, H, Hq, Hkv, d = m["n_layers"], m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    B = len(ctx)
    w = L * (H * (Hq + 2 * Hkv) * d + Hq * d * H)
    if m["n_experts"]:
        w += L * H * m["n_experts"]
        if distinct_experts is None:
            distinct_experts = [min(m["n_experts"], B * m["top_k"])] * L
        w += sum(distinct_experts) * 3 * H * m["expert_ffn"]
    else:
        w += L * 3 * H * m["ffn_dim"]
    w += m["vocab"] * H + B * H + (2 * L + 1) * H
    per_tok = L * 2 * Hkv * d * 2
    kv_read = sum((c + 1) * per_tok for c in ctx)
    kv_write = B * per_tok
    return 2 * w, kv_read, kv_write


def param_counts(m):
    """(total, active) parameter counts; the LM head is untied."""
    L, H, Hq, Hkv, d = m["n_layers"], m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    attn = H * (Hq + 2 * Hkv) * d + Hq * d * H + 2 * H
    if m["n_experts"]:
        ffn_all = H * m["n_experts"] + m["n_experts"] * 3 * H * m["expert_ffn"]
        ffn_act = H * m["n_experts"] + m["top_k"] * 3 * H * m["expert_ffn"]
    else:
        ffn_all = ffn_act = 3 * H * m["ffn_dim"]
    emb = 2 * m["vocab"] * H + H
    return L * (attn + ffn_all) + emb, L * (attn + ffn_act) + emb


def speed_of_light(bytes_per_step, bandwidth):
    """Tokens per second per sequence at a given bandwidth: bandwidth / bytes."""
    return bandwidth / bytes_per_step


# ---------------------------------------------------------------- pool model

class PoolModel:
    """Plain model of the page/slot pool with prefix sharing.

    Pages, slots and leases (kern page, "The runtime": a request leases the
    pages its worst case needs and a state slot, all or nothing): the free
    list is a deque holding the initial page order; a lease takes
    ceil(tokens / page_tokens) pages from the front; slots are the lowest
    free index. Every page records who holds it (sequences, checkpoint
    nodes); it returns to the back of the free list when no one does, a
    finished or released sequence's pages in its page order.

    Prefix sharing (same passage: when a request ends its pages freeze in
    place as a checkpoint; a later request with the same prefix shares the
    whole pages and gets a copy of only the page the prefix ends inside, so
    that every page has at most one writer; a token radix tree finds the
    longest checkpoint for a prompt). Readings: one checkpoint node per page,
    holding the tokens whose K/V the page holds (a tail page holds fewer);
    a run the tree already holds at that place is not frozen twice; the
    reusable prefix of a prompt of n tokens is at most n - 1 tokens (the
    last one runs to give the next token's logits); of equally long matches
    ending inside a page, the earlier checkpoint's page is copied. Under
    pressure (the passage parks checkpoints in host memory; here they are
    dropped) the least recently used checkpoint leaf that no sequence holds
    goes first, ties to the earlier checkpoint; "use" is a lease sharing or
    copying it, or a finish freezing or meeting it, each in path order.
    """

    def __init__(self, order, page_tokens, n_slots):
        self.free = deque(int(p) for p in order)
        self.pt = page_tokens
        self.slots_free = list(range(n_slots))
        self.pages = {}
        self.slot = {}
        self.holders = {int(p): set() for p in order}
        self.nodes = {}          # id -> dict(page, run, parent, made, used)
        self.clock = 0
        self.made = 0

    # -- checkpoints
    def _children(self, parent):
        return sorted((i for i, n in self.nodes.items() if n["parent"] == parent),
                      key=lambda i: self.nodes[i]["made"])

    def _chain(self, i):
        """Node ids from the root's child down to node i."""
        out = []
        while i is not None:
            out.append(i)
            i = self.nodes[i]["parent"]
        return out[::-1]

    def _tokens(self, i):
        return [t for j in self._chain(i) for t in self.nodes[j]["run"]]

    def _use(self, i):
        self.clock += 1
        self.nodes[i]["used"] = self.clock

    def lookup(self, prompt):
        """(tokens reused, node ids shared whole, node copied or None), by
        brute force over every checkpoint's token path."""
        limit = len(prompt) - 1
        if limit <= 0:
            return 0, [], None
        best_m, best = 0, None
        for i in sorted(self.nodes, key=lambda i: self.nodes[i]["made"]):
            path = self._tokens(i)
            c = 0
            while c < min(limit, len(path)) and path[c] == prompt[c]:
                c += 1
            start = len(path) - len(self.nodes[i]["run"])
            if c <= start:
                continue                      # the match ends in an ancestor
            if c > best_m:
                best_m, best = c, i
        if best is None:
            return 0, [], None
        chain = self._chain(best)
        if best_m % self.pt == 0:
            return best_m, chain, None        # the match fills node best's page
        return best_m, chain[:-1], best

    def _evict_one(self):
        leaves = [i for i in self.nodes if not self._children(i)
                  and self.holders[self.nodes[i]["page"]] == {("node", i)}]
        if not leaves:
            return False
        i = min(leaves, key=lambda i: (self.nodes[i]["used"], self.nodes[i]["made"]))
        pg = self.nodes.pop(i)["page"]
        self.holders[pg].clear()
        self.free.append(pg)
        return True

    def _make_free(self, n):
        """Evict until n pages are free; all or nothing."""
        trial = copy.deepcopy(self)
        while len(trial.free) < n:
            if not trial._evict_one():
                return False
        self.__dict__.update(trial.__dict__)
        return True

    # -- leases
    def lease(self, seq, tokens, prompt=None):
        """(slot, tokens reused, copy source page, copy destination page), or
        None when refused (nothing changes then)."""
        if seq in self.pages or not self.slots_free:
            return None
        m, shared, inside = self.lookup(list(prompt)) if prompt is not None else (0, [], None)
        need = -(-tokens // self.pt) - len(shared)
        pinned = [self.nodes[i]["page"] for i in shared + ([inside] if inside is not None else [])]
        for pg in pinned:
            self.holders[pg].add(("pin", seq))
        ok = self._make_free(need)
        for pg in pinned:
            self.holders[pg].discard(("pin", seq))
        if not ok:
            return None
        fresh = [self.free.popleft() for _ in range(need)]
        pages = [self.nodes[i]["page"] for i in shared] + fresh
        for pg in pages:
            self.holders[pg].add(("seq", seq))
        for i in shared:
            self._use(i)
        if inside is not None:
            self._use(inside)
        self.pages[seq] = pages
        self.slots_free.sort()
        self.slot[seq] = self.slots_free.pop(0)
        if inside is None:
            return self.slot[seq], m, -1, -1
        return self.slot[seq], m, self.nodes[inside]["page"], fresh[0]

    def extend(self, seq, tokens):
        need = -(-tokens // self.pt) - len(self.pages[seq])
        if need <= 0:
            return True
        if not self._make_free(need):
            return False
        fresh = [self.free.popleft() for _ in range(need)]
        for pg in fresh:
            self.holders[pg].add(("seq", seq))
        self.pages[seq] += fresh
        return True

    def release(self, seq):
        for pg in self.pages.pop(seq):
            self.holders[pg].discard(("seq", seq))
            if not self.holders[pg]:
                self.free.append(pg)
        self.slots_free.append(self.slot.pop(seq))

    def finish(self, seq, tokens):
        """Freeze seq's pages under its tokens, then release it. Returns
        "ok", "bounds" (more tokens than its pages hold) or "disagree" (a
        page it shares holds other tokens); nothing changes unless "ok"."""
        pages = self.pages[seq]
        runs = [list(tokens[j:j + self.pt]) for j in range(0, len(tokens), self.pt)]
        if len(runs) > len(pages):
            return "bounds"
        frozen = {n["page"] for n in self.nodes.values()}
        parent, on_tree, plan = None, True, []
        for j, run in enumerate(runs):
            hit = None
            if on_tree:
                hit = next((i for i in self._children(parent) if self.nodes[i]["run"] == run), None)
            if hit is None:
                on_tree = False               # below a new node there is nothing to meet
                if pages[j] in frozen:
                    return "disagree"
            plan.append(hit)
            parent = hit
        parent = None
        for j, run in enumerate(runs):
            hit = plan[j]
            if hit is None:
                self.made += 1
                hit = ("n", self.made)
                self.nodes[hit] = dict(page=pages[j], run=run, parent=parent, made=self.made, used=0)
                self.holders[pages[j]].add(("node", hit))
            self._use(hit)
            parent = hit
        self.release(seq)
        return "ok"

    def cached(self):
        return len(self.nodes)

    def page_table(self, seqs, max_pages):
        t = [[-1] * max_pages for _ in seqs]
        for i, s in enumerate(seqs):
            for j, p in enumerate(self.pages[s][:max_pages]):
                t[i][j] = p
        return t


# ---------------------------------------------------------------- work enumeration

def work_sets(m, ctx_bound):
    """What one step must produce, op by op, as sets the plan must cover exactly once.

    Keys: ("qkv", l) rows of W_qkv; ("attn", l) triples (b, kv head, page) for
    the pages that can hold tokens below each sequence's bound; ("comb", l)
    elements (b, q head, dim) of the merged attention output; ("o", l) rows;
    ("router", l) rows; ("gateup", l)
    (b, slot, row) for MoE or rows for dense; ("down", l) rows; ("lm",) rows.

    A batch of several sequences reads each expert's weights once for every
    sequence routed to it, so its expert work is enumerated per expert, for
    any routing: ("router", l) (b, expert row) router logits; ("topk", l)
    sequences; ("gateup", l) (expert, FFN row) and ("down", l) (expert,
    hidden row) over all experts (expert 0 for a dense FFN); ("ffn", l)
    (b, hidden row) of the weighted expert sum.
    """
    L, H, Hq, Hkv, d = m["n_layers"], m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    pt = m["page_tokens"]
    B = len(ctx_bound)
    S = {}
    for l in range(L):
        S["qkv", l] = set(range((Hq + 2 * Hkv) * d))
        S["attn", l] = {(b, g, p) for b in range(B) for g in range(Hkv)
                        for p in range(-(-ctx_bound[b] // pt))}
        S["comb", l] = {(b, h, i) for b in range(B) for h in range(Hq) for i in range(d)}
        S["o", l] = set(range(H))
        if B > 1:
            ne = max(1, m["n_experts"])
            F = m["expert_ffn"] if m["n_experts"] else m["ffn_dim"]
            if m["n_experts"]:
                S["router", l] = {(b, e) for b in range(B) for e in range(m["n_experts"])}
                S["topk", l] = set(range(B))
            S["gateup", l] = {(e, f) for e in range(ne) for f in range(F)}
            S["down", l] = {(e, r) for e in range(ne) for r in range(H)}
            S["ffn", l] = {(b, r) for b in range(B) for r in range(H)}
            continue
        if m["n_experts"]:
            S["router", l] = set(range(m["n_experts"]))
            S["gateup", l] = {(b, j, f) for b in range(B) for j in range(m["top_k"])
                              for f in range(m["expert_ffn"])}
        else:
            S["gateup", l] = set(range(m["ffn_dim"]))
        S["down", l] = set(range(H))
    S["lm", ] = set(range(m["vocab"]))
    return S


# ---------------------------------------------------------------- completion counters

def qkv_row_group(m, r):
    """kv group of row r of W_qkv: q rows by their query head's group (query
    head h uses kv head h // (Hq/Hkv)), then the k rows, then the v rows of
    each kv head."""
    Hq, Hkv, d = m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    if r < Hq * d:
        return (r // d) // (Hq // Hkv)
    if r < (Hq + Hkv) * d:
        return (r - Hq * d) // d
    return (r - (Hq + Hkv) * d) // d


def expected_counters(m, ctx_bound, S=None):
    """Completion count per dependency class and step, from the work alone.

    A finished task adds to its class's counter the number of outputs it
    produced, so after a step each counter has grown by the size of its
    class's share of work_sets, whatever the tiling. Classes (names as
    "op[layer]" or "op[layer][kv head]"): qkv per kv group (rows of W_qkv
    whose head belongs to the group), attn per kv group ((sequence, page)
    pairs of that kv head), comb, o, router, expert (gate/up outputs plus
    down rows), and for a batch topk and ffn; lm for the LM head. Returns
    {name: count}. S: work_sets(m, ctx_bound) if already at hand.
    """
    if S is None:
        S = work_sets(m, ctx_bound)
    L, Hkv = m["n_layers"], m["n_kv_heads"]
    out = {}
    for l in range(L):
        for g in range(Hkv):
            out[f"qkv[{l}][{g}]"] = sum(1 for r in S["qkv", l] if qkv_row_group(m, r) == g)
            out[f"attn[{l}][{g}]"] = sum(1 for (_, gg, _) in S["attn", l] if gg == g)
        out[f"comb[{l}]"] = len(S["comb", l])
        out[f"o[{l}]"] = len(S["o", l])
        if ("router", l) in S:
            out[f"router[{l}]"] = len(S["router", l])
        if ("topk", l) in S:
            out[f"topk[{l}]"] = len(S["topk", l])
        out[f"expert[{l}]"] = len(S["gateup", l]) + len(S["down", l])
        if ("ffn", l) in S:
            out[f"ffn[{l}]"] = len(S["ffn", l])
    out["lm"] = len(S["lm", ])
    return out
