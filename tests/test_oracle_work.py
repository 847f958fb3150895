"""Pins of the oracle's work enumeration, completion counts and routing rule.

- work_sets against enumerations written out by hand for tiny models (a
  dense decoder, a batch-1 MoE and a batch MoE), and against closed-form
  cardinalities at the 48-layer shapes;
- expected_counters: each class's count is the size of its share of the
  work, written here as closed forms (rows of W_qkv per kv group are its
  query heads' rows plus one k and one v head; pages per kv head are the
  pages below each sequence's bound);
- near_tie, ids_near_tie and decode_step_following: an exact tie between
  two experts (identical router rows) is a near-tie, at the k-th slot and
  inside the selection (the same two experts in the other order), and
  following the other side's choice there equals a step with those ids
  forced; a disagreement away from a tie is reported, not followed.
"""
import itertools

import torch

import oracle as O
from fixtures import HostKV, HostWeights, workload


def tiny(**over):
    m = dict(n_layers=1, hidden=16, n_q_heads=2, n_kv_heads=1, head_dim=4, ffn_dim=8,
             n_experts=0, top_k=0, expert_ffn=0, norm_topk=1, vocab=5, page_tokens=16,
             rms_eps=1e-6, rope_theta=1e4)
    m.update(over)
    return m


def test_work_sets_dense_by_hand():
    # one layer, bound 17: tokens 0 .. 16 need pages 0 and 1
    S = O.work_sets(tiny(), [17])
    assert S["qkv", 0] == set(range(16))                 # (2 + 2 * 1) heads x 4 dims
    assert S["attn", 0] == {(0, 0, 0), (0, 0, 1)}
    assert S["comb", 0] == {(0, h, i) for h in (0, 1) for i in (0, 1, 2, 3)}
    assert S["o", 0] == set(range(16))
    assert S["gateup", 0] == set(range(8))
    assert S["down", 0] == set(range(16))
    assert S["lm", ] == {0, 1, 2, 3, 4}
    assert set(S) == {("qkv", 0), ("attn", 0), ("comb", 0), ("o", 0), ("gateup", 0), ("down", 0), ("lm", )}
    # bound 16 fits one page; bound 1 still needs page 0
    assert O.work_sets(tiny(), [16])["attn", 0] == {(0, 0, 0)}
    assert O.work_sets(tiny(), [1])["attn", 0] == {(0, 0, 0)}


def test_work_sets_moe_batch1_by_hand():
    m = tiny(n_experts=4, top_k=2, expert_ffn=2, ffn_dim=0)
    S = O.work_sets(m, [33])
    assert S["attn", 0] == {(0, 0, 0), (0, 0, 1), (0, 0, 2)}
    assert S["router", 0] == {0, 1, 2, 3}
    # (sequence, slot, FFN row): the two routed slots, whichever experts they hold
    assert S["gateup", 0] == {(0, 0, 0), (0, 0, 1), (0, 1, 0), (0, 1, 1)}
    assert S["down", 0] == set(range(16))


def test_work_sets_moe_batch_by_hand():
    # a batch reads each expert once for all sequences routed to it: expert
    # work is enumerated per expert, for any routing
    m = tiny(n_experts=4, top_k=2, expert_ffn=2, ffn_dim=0, n_kv_heads=2, n_q_heads=2)
    S = O.work_sets(m, [5, 20])
    assert S["attn", 0] == {(0, 0, 0), (0, 1, 0), (1, 0, 0), (1, 0, 1), (1, 1, 0), (1, 1, 1)}
    assert S["router", 0] == {(b, e) for b in (0, 1) for e in range(4)}
    assert S["topk", 0] == {0, 1}
    assert S["gateup", 0] == {(e, f) for e in range(4) for f in (0, 1)}
    assert S["down", 0] == {(e, r) for e in range(4) for r in range(16)}
    assert S["ffn", 0] == {(b, r) for b in (0, 1) for r in range(16)}
    assert S["comb", 0] == {(b, h, i) for b in (0, 1) for h in (0, 1) for i in range(4)}
    assert S["qkv", 0] == set(range(24))                 # (2 + 2 * 2) heads x 4 dims


def test_work_sets_cardinalities_at_moe48():
    m = workload("moe48_b1_8k")["model"]
    L, H, Hq, Hkv, d = 48, 2048, 32, 4, 128
    S = O.work_sets(m, [8192 + 256])
    pages = -(-(8192 + 256) // 16)
    for l in (0, 47):
        assert len(S["qkv", l]) == (Hq + 2 * Hkv) * d == 5120
        assert len(S["attn", l]) == Hkv * pages == 4 * 528
        assert len(S["comb", l]) == Hq * d
        assert len(S["o", l]) == H
        assert len(S["router", l]) == 128
        assert len(S["gateup", l]) == 8 * 768
        assert len(S["down", l]) == H
    assert len(S["lm", ]) == 151936
    assert len(S) == 7 * L + 1


def test_expected_counters_closed_forms():
    m = workload("moe48_b1_8k")["model"]
    bound = 8192 + 256
    c = O.expected_counters(m, [bound])
    pages = -(-bound // 16)
    for l in (0, 23, 47):
        for g in range(4):
            assert c[f"qkv[{l}][{g}]"] == (32 // 4 + 2) * 128     # 8 query heads, one k, one v
            assert c[f"attn[{l}][{g}]"] == pages
        assert c[f"comb[{l}]"] == 32 * 128
        assert c[f"o[{l}]"] == 2048
        assert c[f"router[{l}]"] == 128
        assert c[f"expert[{l}]"] == 8 * 768 + 2048
    assert c["lm"] == 151936
    assert len(c) == 48 * (2 * 4 + 4) + 1
    # a batch: per-sequence pages, every expert, top-k and combine per sequence
    ctx = [100, 16, 5000]
    cb = O.expected_counters(m, ctx)
    for g in range(4):
        assert cb[f"attn[3][{g}]"] == sum(-(-x // 16) for x in ctx)
    assert cb["router[3]"] == 3 * 128 and cb["topk[3]"] == 3 and cb["ffn[3]"] == 3 * 2048
    assert cb["expert[3]"] == 128 * (768 + 2048) and cb["comb[3]"] == 3 * 32 * 128


def test_qkv_row_groups_follow_the_gqa_mapping():
    m = tiny(n_q_heads=4, n_kv_heads=2)                  # heads 0, 1 -> group 0; 2, 3 -> group 1
    groups = [O.qkv_row_group(m, r) for r in range((4 + 4) * 4)]
    assert groups == [0] * 8 + [1] * 8 + [0] * 4 + [1] * 4 + [0] * 4 + [1] * 4


def test_near_tie_rule():
    r = torch.tensor([1.0, 3.0, 2.0, 2.0])
    assert O.near_tie(r, 2, 1e-5)                        # 2nd and 3rd probabilities equal
    assert not O.near_tie(r, 1, 1e-5)
    assert not O.near_tie(torch.tensor([3.0, 2.0, 1.0]), 2, 1e-5)
    assert O.near_tie(torch.tensor([3.0, 2.0, 2.0 - 1e-7]), 2, 1e-5)


def tied_moe(k):
    """A 2-layer MoE (top-k) whose router rows 1 and 2 are identical and rows
    0 and 3 zero in every layer: the logits are (0, a, a, 0), so experts 1
    and 2 tie, and so do experts 0 and 3."""
    m = tiny(n_layers=2, hidden=32, n_q_heads=2, n_kv_heads=1, head_dim=16, ffn_dim=0,
             n_experts=4, top_k=k, expert_ffn=32, vocab=50)
    W = HostWeights(m, seed=11)
    for l in range(2):
        r = W.router(l)
        r[2] = r[1]
        r[0] = 0
        r[3] = 0
    return m, W


def partner(e):
    return {0: 3, 3: 0, 1: 2, 2: 1}[e]


def test_following_an_exact_tie_equals_forcing_it():
    m, W = tied_moe(1)
    kv = O.OracleKV(m, [7], 2, HostKV(m, seed=11))
    base = O.decode_step(m, W, kv, [3])
    e0 = int(base["topk_ids"][0][0][0])
    assert e0 in (0, 1)                                  # equal probabilities: the lower index
    assert O.near_tie(base["router_logits"][0][0], 1, 1e-5)
    # the other side ranked the tied pair the other way at layer 0
    other = [[[partner(e0)], [int(base["topk_ids"][0][1][0])]]]
    kv.len = [7]
    out, forced, differ = O.decode_step_following(m, W, kv, [3], other, 1e-5)
    assert forced == [(0, 0)] and differ == []
    kv2 = O.OracleKV(m, [7], 2, HostKV(m, seed=11))
    want = O.decode_step(m, W, kv2, [3], force_ids={(0, 0): [partner(e0)]})
    assert torch.equal(out["x_ffn"][0][0], want["x_ffn"][0][0])
    assert torch.equal(out["logits"][0], want["logits"][0])
    assert not torch.equal(out["x_ffn"][0][0], base["x_ffn"][0][0])


def test_following_does_not_hide_a_real_difference():
    m, W = tied_moe(2)
    kv = O.OracleKV(m, [7], 2, HostKV(m, seed=11))
    own = O.decode_step(m, W, kv, [3])
    ids = own["topk_ids"][0][0].tolist()
    assert ids in ([1, 2], [0, 3])
    assert not O.near_tie(own["router_logits"][0][0], 2, 1e-5)
    other = [[[0, 3] if ids == [1, 2] else [1, 2], own["topk_ids"][0][1].tolist()]]
    kv.len = [7]
    out, forced, differ = O.decode_step_following(m, W, kv, [3], other, 1e-5)
    assert forced == [] and differ == [(0, 0)]
    # agreeing ids change nothing
    kv.len = [7]
    same = [[own["topk_ids"][0][l].tolist() for l in range(2)]]
    out2, forced2, differ2 = O.decode_step_following(m, W, kv, [3], same, 1e-5)
    assert forced2 == [] and differ2 == [] and torch.equal(out2["logits"][0], own["logits"][0])


def test_following_an_order_swap_inside_the_selection():
    # top-2 of (0, a, a, 0): experts 1 and 2 are both selected and tie, so
    # the other order of the same two experts is a near-tie and is followed
    m, W = tied_moe(2)
    kv = O.OracleKV(m, [7], 2, HostKV(m, seed=11))
    own = O.decode_step(m, W, kv, [3])
    ids = own["topk_ids"][0][0].tolist()
    assert sorted(ids) in ([1, 2], [0, 3])
    swapped = ids[::-1]
    assert O.ids_near_tie(own["router_logits"][0][0], ids, swapped, 1e-5)
    other = [[swapped, own["topk_ids"][0][1].tolist()]]
    kv.len = [7]
    out, forced, differ = O.decode_step_following(m, W, kv, [3], other, 1e-5)
    assert forced == [(0, 0)] and differ == []
    kv2 = O.OracleKV(m, [7], 2, HostKV(m, seed=11))
    want = O.decode_step(m, W, kv2, [3], force_ids={(0, 0): swapped})
    assert torch.equal(out["x_ffn"][0][0], want["x_ffn"][0][0])
    assert torch.equal(out["logits"][0], want["logits"][0])


def test_ids_near_tie_rule():
    r = torch.tensor([1.0, 3.0, 2.0, 2.0, 0.5])
    assert O.ids_near_tie(r, [1, 2], [1, 3], 1e-5)      # k-th and (k+1)-th equal
    assert O.ids_near_tie(r, [1, 2, 3], [1, 3, 2], 1e-5)  # equal pair inside the selection
    assert not O.ids_near_tie(r, [1, 2], [2, 1], 1e-5)  # 3.0 and 2.0 are far apart
    assert not O.ids_near_tie(r, [1, 2], [1, 0], 1e-5)
    assert O.ids_near_tie(r, [1, 2], [1, 2], 0.0)       # equal lists
    # relative threshold: logits 0 and -1e-6 give probabilities about 1e-6 apart
    q = torch.tensor([0.0, -1e-6, -5.0])
    assert O.ids_near_tie(q, [0, 1], [1, 0], 1e-5) and not O.ids_near_tie(q, [0, 1], [1, 0], 1e-7)


def test_forced_weights_are_the_renormalised_probabilities():
    r = torch.tensor([0.3, -1.0, 2.0, 0.7], dtype=torch.float64)
    ids, w = O.route_given(r, [3, 0])
    p = torch.softmax(r, dim=0)
    assert ids.tolist() == [3, 0]
    assert torch.allclose(w, torch.stack([p[3], p[0]]) / (p[3] + p[0]), rtol=1e-15)
    # the forced form of the oracle's own choice equals its own routing
    ids2, w2 = O.route(r, 2)
    ids3, w3 = O.route_given(r, ids2.tolist())
    assert torch.equal(ids2, ids3) and torch.equal(w2, w3)
    for perm in itertools.permutations(range(4), 2):
        _, wp = O.route_given(r, list(perm))
        assert abs(float(wp.sum()) - 1.0) < 1e-15
