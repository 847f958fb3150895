"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks an oracle function against something other than itself:
a brute-force fp64 evaluation in plain Python loops on tiny inputs, a
closed form, an invariant, or a special case that reduces to a simpler
routine. Planted-mistake tests at the end show that plausible errors
(a dropped term, a wrong sign, a transposed operand) fail a pin.
"""
import math
import random

import pytest
import torch

import oracle as O
from fixtures import HostWeights, HostKV, workload

torch.manual_seed(0)


def bf16(t):
    return t.to(torch.bfloat16)


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    for c in (0.5, -3.0, 1e-3):
        x = torch.full((64,), c, dtype=torch.float64)
        g = bf16(torch.ones(64))
        y = O.rmsnorm(x, g, 1e-6)
        want = c / math.sqrt(c * c + 1e-6)
        assert torch.allclose(y, torch.full_like(y, want), rtol=1e-14, atol=0)


def test_rmsnorm_brute_force_and_scale_invariance():
    x = torch.randn(37, dtype=torch.float64)
    g = bf16(torch.rand(37) + 0.5)
    y = O.rmsnorm(x, g, 1e-6)
    ms = math.fsum(v * v for v in x.tolist()) / 37
    for i in range(37):
        assert abs(y[i].item() - x[i].item() / math.sqrt(ms + 1e-6) * g[i].float().item()) < 1e-13
    y2 = O.rmsnorm(1000.0 * x, g, 0.0)
    assert torch.allclose(O.rmsnorm(x, g, 0.0), y2, rtol=1e-13, atol=0)


# ------------------------------------------------------------------ projections

def test_matvec_f64_dot_and_identity():
    W = bf16(torch.randn(19, 45))
    u = torch.randn(45, dtype=torch.float64)
    y = O.matvec(W, u)
    Wf = W.double().tolist()
    for r in range(19):
        ref = math.fsum(Wf[r][c] * u[c].item() for c in range(45))
        assert abs(y[r].item() - ref) < 1e-12
    eye = bf16(torch.eye(45))
    assert torch.equal(O.matvec(eye, u), u)
    # a non-square matrix catches a transposed operand
    assert y.shape == (19,)


def test_batch_row_equals_single_row():
    W = HostWeights(workload("tiny_dense")["model"], seed=3)
    m = W.m
    kv1 = O.OracleKV(m, [20, 33], 4, HostKV(m, seed=3))
    kv2 = O.OracleKV(m, [33], 4, None)
    for l in range(m["n_layers"]):
        for g in range(m["n_kv_heads"]):
            kv2.K[l, 0, g][:33] = kv1.K[l, 1, g][:33]
            kv2.V[l, 0, g][:33] = kv1.V[l, 1, g][:33]
    a = O.decode_step(m, W, kv1, [5, 77])
    b = O.decode_step(m, W, kv2, [77])
    assert torch.equal(a["logits"][1], b["logits"][0])


# ------------------------------------------------------------------ RoPE

def test_rope_position_zero_is_identity():
    c, s = O.rope_cos_sin(1e4, 64, 0)
    v = torch.randn(3, 64)
    assert torch.equal(O.rope(v, c, s), v)


def test_rope_preserves_pair_norms():
    c, s = O.rope_cos_sin(1e4, 64, 1234)
    v = torch.randn(5, 64, dtype=torch.float64)
    r = O.rope(v, c, s)
    n0 = v[:, :32] ** 2 + v[:, 32:] ** 2
    n1 = r[:, :32] ** 2 + r[:, 32:] ** 2
    assert torch.allclose(n0, n1, rtol=1e-6)


def test_rope_relative_position_and_composition():
    d = 64
    q = torch.randn(d, dtype=torch.float64)
    k = torch.randn(d, dtype=torch.float64)

    def R(p, v):
        c, s = O.rope_cos_sin(1e4, d, p)
        return O.rope(v[None], c.double(), s.double())[0]

    dots = [float(R(p + 7, q) @ R(p, k)) for p in (0, 100, 5000)]
    assert max(dots) - min(dots) < 1e-5 * max(1.0, abs(dots[0]))
    # R(a) R(b) = R(a + b) up to fp32 rounding of the table
    assert torch.allclose(R(300, R(45, q)), R(345, q), atol=1e-5)


def test_rope_table_is_fp32_rounding_of_fp64():
    c, s = O.rope_cos_sin(1e4, 128, 262143)
    assert c.dtype == torch.float32
    i = 17
    ang = 262143 * (1e4 ** (-2 * i / 128))
    assert c[i].item() == float(torch.tensor(math.cos(ang), dtype=torch.float32))
    assert s[i].item() == float(torch.tensor(math.sin(ang), dtype=torch.float32))


# ------------------------------------------------------------------ attention

def brute_attention(q, K, V):
    """fp64 softmax attention in plain Python loops."""
    n, d = len(q), len(q[0])
    out = []
    for h in range(n):
        s = [math.fsum(q[h][i] * K[j][i] for i in range(d)) / math.sqrt(d) for j in range(len(K))]
        mx = max(s)
        e = [math.exp(v - mx) for v in s]
        z = math.fsum(e)
        out.append([math.fsum(e[j] * V[j][i] for j in range(len(K))) / z for i in range(d)])
    return out


@pytest.mark.parametrize("T", [1, 5, 16, 17, 48])
def test_attention_brute_force(T):
    d = 4
    q = torch.randn(3, d, dtype=torch.float64)
    K = bf16(torch.randn(T, d))
    V = bf16(torch.randn(T, d))
    o = O.attention(q, K, V)
    ref = brute_attention(q.tolist(), K.double().tolist(), V.double().tolist())
    assert torch.allclose(o, torch.tensor(ref, dtype=torch.float64), atol=1e-13)


def test_attention_special_cases():
    d = 8
    q = torch.randn(2, d, dtype=torch.float64)
    K = bf16(torch.randn(1, d)).repeat(10, 1)  # all keys equal: mean of V
    V = bf16(torch.randn(10, d))
    assert torch.allclose(O.attention(q, K, V)[0], V.double().mean(0), atol=1e-12)
    K = bf16(torch.zeros(10, d))
    K[6] = 1.0
    qq = torch.full((1, d), 200.0, dtype=torch.float64)  # one dominant score
    assert torch.allclose(O.attention(qq, K, V)[0], V[6].double(), atol=1e-12)


def test_paged_equals_contiguous_and_page_shuffle_invariance():
    pt, d, n_tok = 16, 8, 53
    n_pg = -(-n_tok // pt)
    K = bf16(torch.randn(n_pg * pt, d))
    V = bf16(torch.randn(n_pg * pt, d))
    q = torch.randn(4, d)
    ref = O.attention(q, K[:n_tok], V[:n_tok])
    for seed in range(3):
        rng = random.Random(seed)
        n_pool = 11
        phys = rng.sample(range(n_pool), n_pg)
        pool_k = bf16(torch.randn(n_pool, pt, d))
        pool_v = bf16(torch.randn(n_pool, pt, d))
        for j, p in enumerate(phys):
            pool_k[p] = K[j * pt:(j + 1) * pt]
            pool_v[p] = V[j * pt:(j + 1) * pt]
        got = O.attention_paged(q, pool_k, pool_v, phys, n_tok, pt)
        assert torch.equal(got, ref)


def test_split_merge_equals_single_pass():
    d, T = 16, 200
    q = torch.randn(8, d, dtype=torch.float64)
    K = bf16(torch.randn(T, d) * 3)
    V = bf16(torch.randn(T, d))
    ref = O.attention(q, K, V)
    for cuts in ([0, 200], [0, 16, 64, 200], [0, 1, 2, 199, 200]):
        parts = [O.attention_partial(q, K[a:b], V[a:b]) for a, b in zip(cuts, cuts[1:])]
        assert torch.allclose(O.merge_partials(parts), ref, atol=1e-12, rtol=0)


# ------------------------------------------------------------------ router / MoE / argmax

def test_topk_brute_force_with_ties():
    for trial in range(50):
        rng = random.Random(trial)
        p = torch.tensor([rng.choice([0.1, 0.2, 0.3, rng.random()]) for _ in range(32)])
        k = rng.randint(1, 32)
        want = sorted(range(32), key=lambda i: (-p[i].item(), i))[:k]
        assert O.topk(p, k).tolist() == want


def test_route_identities():
    r = torch.randn(32, dtype=torch.float64)
    ids, w = O.route(r, 32)
    assert sorted(ids.tolist()) == list(range(32))
    assert torch.allclose(w, O.softmax(r)[ids], rtol=1e-14)  # k = E: plain softmax
    ids, w = O.route(r, 5)
    # renormalised top-k == softmax over the selected logits
    assert torch.allclose(w, O.softmax(r[ids]), rtol=1e-13)
    assert ids.tolist() == sorted(range(32), key=lambda i: -r[i].item())[:5]


class Tiny:
    """Explicit small weights with the HostWeights accessor interface."""

    def __init__(self, m, gen, identical_experts=False):
        self.m = m
        H, Hq, Hkv, d, V = m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"], m["vocab"]
        L = m["n_layers"]
        f = m["expert_ffn"] if m["n_experts"] else m["ffn_dim"]
        E = max(1, m["n_experts"])
        r = lambda *s: bf16(torch.randn(*s, generator=gen) * 0.3)
        self.E = r(V, H)
        self.qkv = [r((Hq + 2 * Hkv) * d, H) for _ in range(L)]
        self.o = [r(H, Hq * d) for _ in range(L)]
        self.r = [r(E, H) for _ in range(L)]
        g0, u0, d0 = r(f, H), r(f, H), r(H, f)
        self.g = [[g0 if identical_experts else r(f, H) for _ in range(E)] for _ in range(L)]
        self.u = [[u0 if identical_experts else r(f, H) for _ in range(E)] for _ in range(L)]
        self.dn = [[d0 if identical_experts else r(H, f) for _ in range(E)] for _ in range(L)]
        self.lm = r(V, H)

    def embed_row(self, t): return self.E[t]
    def attn_norm(self, l): return bf16(torch.ones(self.m["hidden"]))
    ffn_norm = attn_norm
    def final_norm(self): return bf16(torch.ones(self.m["hidden"]))
    def wqkv(self, l): return self.qkv[l]
    def wo(self, l): return self.o[l]
    def router(self, l): return self.r[l]
    def gate(self, l, e=0): return self.g[l][e]
    def up(self, l, e=0): return self.u[l][e]
    def down(self, l, e=0): return self.dn[l][e]
    def lm_head(self): return self.lm


TINY = dict(n_layers=2, hidden=16, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn_dim=0,
            n_experts=6, top_k=3, expert_ffn=12, norm_topk=1, vocab=40, page_tokens=16,
            rms_eps=1e-6, rope_theta=1e4)


def test_identical_experts_equal_dense_swiglu():
    gen = torch.Generator().manual_seed(1)
    moe = Tiny(TINY, gen, identical_experts=True)
    dense_m = dict(TINY, n_experts=0, top_k=0, expert_ffn=0, ffn_dim=12)
    dense = Tiny(dense_m, torch.Generator().manual_seed(1))
    for name in ("E", "qkv", "o", "lm"):
        setattr(dense, name, getattr(moe, name))
    dense.g = [[moe.g[l][0]] for l in range(2)]
    dense.u = [[moe.u[l][0]] for l in range(2)]
    dense.dn = [[moe.dn[l][0]] for l in range(2)]
    a = O.decode_step(TINY, moe, O.OracleKV(TINY, [5], 2, None), [3], dt=torch.float64)
    b = O.decode_step(dense_m, dense, O.OracleKV(dense_m, [5], 2, None), [3], dt=torch.float64)
    assert torch.allclose(a["logits"][0], b["logits"][0], atol=1e-12)


def test_k1_routes_to_the_argmax_expert_with_weight_one():
    m = dict(TINY, top_k=1)
    W = Tiny(m, torch.Generator().manual_seed(2))
    out = O.decode_step(m, W, O.OracleKV(m, [4], 2, None), [7], dt=torch.float64)
    for l in range(2):
        assert out["topk_w"][0][l].tolist() == [1.0]
        assert out["topk_ids"][0][l].item() == int(torch.argmax(out["router_logits"][0][l]))


def test_argmax_ties_lower_index():
    v = torch.tensor([0.1, 0.7, 0.3, 0.7, 0.7])
    assert O.argmax(v) == 1
    for trial in range(30):
        rng = random.Random(trial)
        v = torch.tensor([float(rng.randint(0, 5)) for _ in range(50)])
        assert O.argmax(v) == min(i for i in range(50) if v[i] == v.max())


# ------------------------------------------------------------------ whole step

def brute_step(m, W, Kc, Vc, tok):
    """Whole step for one sequence in fp64 plain Python loops (tiny shapes only).

    Kc[l][g], Vc[l][g]: lists of prior key/value rows (floats).
    """
    H, Hq, Hkv, d = m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    eps, hg = m["rms_eps"], Hq // Hkv

    def mv(w, u):
        wl = w.double().tolist()
        return [math.fsum(wl[r][c] * u[c] for c in range(len(u))) for r in range(len(wl))]

    def norm(x):
        s = math.sqrt(math.fsum(v * v for v in x) / len(x) + eps)
        return [v / s for v in x]

    def rot(v, p):
        out = list(v)
        for i in range(d // 2):
            a = p * m["rope_theta"] ** (-2 * i / d)
            c, s = float(torch.tensor(math.cos(a)).float()), float(torch.tensor(math.sin(a)).float())
            out[i] = v[i] * c - v[i + d // 2] * s
            out[i + d // 2] = v[i + d // 2] * c + v[i] * s
        return out

    def r16(v):
        return [float(torch.tensor(t, dtype=torch.float32).to(torch.bfloat16)) for t in v]

    pos = len(Kc[0][0])
    x = W.embed_row(tok).double().tolist()
    for l in range(m["n_layers"]):
        qkv = mv(W.wqkv(l), norm(x))
        q = [rot(qkv[h * d:(h + 1) * d], pos) for h in range(Hq)]
        k = [r16(rot(qkv[(Hq + g) * d:(Hq + g + 1) * d], pos)) for g in range(Hkv)]
        v = [r16(qkv[(Hq + Hkv + g) * d:(Hq + Hkv + g + 1) * d]) for g in range(Hkv)]
        o = []
        for h in range(Hq):
            g = h // hg
            o += brute_attention([q[h]], Kc[l][g] + [k[g]], Vc[l][g] + [v[g]])[0]
        y = mv(W.wo(l), o)
        x = [a + b for a, b in zip(x, y)]
        u = norm(x)
        r = mv(W.router(l), u)
        mx = max(r)
        e = [math.exp(t - mx) for t in r]
        p = [t / math.fsum(e) for t in e]
        ids = sorted(range(len(p)), key=lambda i: (-p[i], i))[: m["top_k"]]
        wsum = math.fsum(p[i] for i in ids)
        acc = [0.0] * H
        for i in ids:
            gg, uu = mv(W.gate(l, i), u), mv(W.up(l, i), u)
            a = [s / (1 + math.exp(-s)) * t for s, t in zip(gg, uu)]
            dn = mv(W.down(l, i), a)
            acc = [s + p[i] / wsum * t for s, t in zip(acc, dn)]
        x = [s + t for s, t in zip(x, acc)]
    return mv(W.lm_head(), norm(x))


def test_whole_step_brute_force_tiny_moe():
    m = TINY
    W = Tiny(m, torch.Generator().manual_seed(4))
    ctx = 21
    kv = O.OracleKV(m, [ctx], 2, None)
    Kc = [[[] for _ in range(2)] for _ in range(2)]
    Vc = [[[] for _ in range(2)] for _ in range(2)]
    for l in range(2):
        for g in range(2):
            K = bf16(torch.randn(ctx, 8))
            V = bf16(torch.randn(ctx, 8))
            kv.K[l, 0, g][:ctx] = K
            kv.V[l, 0, g][:ctx] = V
            Kc[l][g] = K.double().tolist()
            Vc[l][g] = V.double().tolist()
    out = O.decode_step(m, W, kv, [11], dt=torch.float64)
    ref = brute_step(m, W, Kc, Vc, 11)
    assert torch.allclose(out["logits"][0], torch.tensor(ref, dtype=torch.float64), atol=1e-9)


def test_reduces_to_embedding_when_branches_are_zero():
    m = TINY
    W = Tiny(m, torch.Generator().manual_seed(5))
    W.o = [bf16(torch.zeros_like(w.float())) for w in W.o]
    W.dn = [[bf16(torch.zeros_like(w.float())) for w in row] for row in W.dn]
    out = O.decode_step(m, W, O.OracleKV(m, [3], 2, None), [9], dt=torch.float64)
    x = W.E[9].double()
    z = x / torch.sqrt((x * x).mean() + m["rms_eps"])
    assert torch.allclose(out["logits"][0], W.lm.double() @ z, atol=1e-12)


def test_fp32_and_fp64_modes_agree_and_determinism():
    w = workload("tiny_dense")
    m = w["model"]
    W = HostWeights(m, seed=0)
    res = {}
    for dt in (torch.float32, torch.float64):
        kv = O.OracleKV(m, w["ctx"], 4, HostKV(m, seed=0))
        res[dt] = O.decode_step(m, W, kv, [17], dt=dt)
    for l in range(m["n_layers"]):
        a, b = res[torch.float32]["x_ffn"][0][l].double(), res[torch.float64]["x_ffn"][0][l]
        assert (a - b).abs().max() / b.abs().max() < 1e-4
    kv = O.OracleKV(m, w["ctx"], 4, HostKV(m, seed=0))
    again = O.decode_step(m, W, kv, [17])
    assert torch.equal(again["logits"][0], res[torch.float32]["logits"][0])


# ------------------------------------------------------------------ planted mistakes

def test_planted_mistakes_fail_a_pin(monkeypatch):
    """Each plausible mistake in the oracle breaks the brute-force whole-step pin."""
    m = TINY
    W = Tiny(m, torch.Generator().manual_seed(6))
    kv0 = O.OracleKV(m, [9], 2, None)
    Kc = [[[] for _ in range(2)] for _ in range(2)]
    Vc = [[[] for _ in range(2)] for _ in range(2)]
    for l in range(2):
        for g in range(2):
            K, V = bf16(torch.randn(9, 8)), bf16(torch.randn(9, 8))
            kv0.K[l, 0, g][:9], kv0.V[l, 0, g][:9] = K, V
            Kc[l][g], Vc[l][g] = K.double().tolist(), V.double().tolist()
    ref = torch.tensor(brute_step(m, W, Kc, Vc, 2), dtype=torch.float64)

    def run():
        kv = O.OracleKV(m, [9], 2, None)
        for key in kv0.K:
            kv.K[key].copy_(kv0.K[key])
            kv.V[key].copy_(kv0.V[key])
        return O.decode_step(m, W, kv, [2], dt=torch.float64)["logits"][0]

    assert torch.allclose(run(), ref, atol=1e-9)
    good_rope, good_mv, good_rms, good_soft = O.rope, O.matvec, O.rmsnorm, O.softmax
    mistakes = {
        "rope sign": lambda v, c, s: good_rope(v, c, -s),
        "adjacent rope pairs": lambda v, c, s: torch.stack(
            [v[..., 0::2] * c.to(v.dtype) - v[..., 1::2] * s.to(v.dtype),
             v[..., 1::2] * c.to(v.dtype) + v[..., 0::2] * s.to(v.dtype)], -1).reshape(v.shape),
    }
    for name, bad in mistakes.items():
        monkeypatch.setattr(O.oracle, "rope", bad)
        assert not torch.allclose(run(), ref, atol=1e-6), name
        monkeypatch.setattr(O.oracle, "rope", good_rope)
    monkeypatch.setattr(O.oracle, "rmsnorm", lambda x, g, eps: x / torch.sqrt((x * x).sum() + eps))
    assert not torch.allclose(run(), ref, atol=1e-6)
    monkeypatch.setattr(O.oracle, "rmsnorm", good_rms)
    monkeypatch.setattr(O.oracle, "softmax", lambda s: torch.exp(s) / torch.exp(s).sum(-1, keepdim=True) * 1.01)
    assert not torch.allclose(run(), ref, atol=1e-6)
    monkeypatch.setattr(O.oracle, "softmax", good_soft)
    monkeypatch.setattr(O.oracle, "route", lambda r, k, n=True: (O.topk(r, k), torch.ones(k, dtype=r.dtype) / k))
    assert not torch.allclose(run(), ref, atol=1e-6)
