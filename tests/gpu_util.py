"""Shared helpers of the GPU parity tests (comparison metrics and triage)."""
import torch

import oracle as O

# Hidden-state tolerance: max |gpu - oracle| / max |oracle| over a vector.
HIDDEN_TOL = 2e-2
# Regression guard: the kernels' hidden states and logits land within about
# 2e-4 of the oracle (fp32 accumulation throughout); an error ten times that,
# though inside HIDDEN_TOL, means an accuracy regression and fails.
REGRESSION_TOL = 2e-3
# A top-k or argmax disagreement is a near-tie (reported, not failed) when
# the oracle's two competing scores differ by less than this fraction. The
# decision is taken in fp32 on both sides, on inputs that differ by the
# accumulated rounding of the layers before it: at the 48th layer hidden
# states and router logits sit about 1e-4 (relative) from the oracle's, and
# logits that far apart can swap two probabilities whose ratio is within
# about 2e-4 of 1. The threshold leaves a margin of five over that.
NEAR_TIE = 1e-3


def rel_err(got, want):
    got = got.detach().double().cpu().reshape(-1)
    want = want.detach().double().cpu().reshape(-1)
    den = want.abs().max().item()
    return (got - want).abs().max().item() / (den if den > 0 else 1.0)


def topk_near_tie(router_logits, k):
    """True when the oracle's k-th and (k+1)-th router probabilities nearly tie."""
    p = torch.softmax(router_logits.double(), dim=-1)
    s = torch.sort(p, descending=True).values
    if k >= s.numel():
        return False
    return (s[k - 1] - s[k]).item() < NEAR_TIE * s[k - 1].item()


def argmax_near_tie(logits, a, b):
    """True when logits a and b (two candidate ids) nearly tie."""
    la, lb = float(logits[a]), float(logits[b])
    return abs(la - lb) < NEAR_TIE * max(abs(la), abs(lb), 1.0)


def flush(msg):
    print(msg, flush=True)


def kv_offsets(s, d):
    """Element offsets, within one (page, layer, kv head) block of the KV pool,
    of K[s][0..d) and V[s][0..d) for token slot s, in the pool's documented
    operand order."""
    dim = torch.arange(d)
    k = (((dim // 32) * 4 + (dim % 32) // 8) * 16 + s) * 8 + dim % 8
    v = 16 * d + (((dim // 32) * 4 + s // 4) * 16 + dim % 16) * 8 + ((dim % 32) // 16) * 4 + s % 4
    return k, v


def plan_bounds(w):
    """Context bounds a workload's plan covers, as the oracle's work
    enumeration takes them: one bound at batch 1, one per sequence in a batch."""
    if w["batch"] > 1:
        return [c + w["steps"] for c in w["ctx"]]
    return [max(w["ctx"]) + w["steps"]]


def check_counters_against_oracle(names, values, exp, steps=1):
    """values[i] (counter names[i]) == steps x the oracle's count of its class,
    modulo 2^32. A per-layer name of a class the oracle counts per kv group
    sums the groups (queued attention: one counter per layer); queue heads
    are the plan's own bookkeeping and are skipped."""
    seen = set()
    for nm, v in zip(names, values):
        if nm.startswith("queue["):
            continue
        if nm in exp:
            want = exp[nm]
            seen.add(nm)
        else:
            parts = [k for k in exp if k.startswith(nm + "[")]
            assert parts, f"counter {nm} has no class in the oracle"
            want = sum(exp[k] for k in parts)
            seen.update(parts)
        assert int(v) % (1 << 32) == (steps * want) % (1 << 32), f"counter {nm}: {int(v)} != {steps} x {want}"
    assert seen == set(exp), f"classes without a counter: {sorted(set(exp) - seen)[:5]}"


def check_device_counters(dec, w):
    """The device's completion counters after dec.epoch steps equal the
    oracle's completion count of each class times the steps."""
    import decode_megakernel_persistent_amd as mk
    exp = O.expected_counters(w["model"], plan_bounds(w))
    check_counters_against_oracle(mk.mk_plan_counter_names(dec.plan), dec.counters().tolist(), exp,
                                  steps=dec.epoch)


def gpu_routing(ids, b):
    """[layer][k] expert ids of sequence b from a device [L][B][k] tensor."""
    return [[int(v) for v in row] for row in ids[:, b].cpu().tolist()]


def compare_sequence(dec, m, b, ref, rb, ids=None, tw=None, logits=None, tok_out=None, pos=None, pool_slot=None,
                     layers=None):
    """GPU sequence b against row rb of an oracle result (decode_step or
    decode_step_following on the GPU's routing): top-k ids bit-exact, top-k
    weights, router logits, hidden state after every attention and FFN
    residual, the new K and V in the pool, the logits, the next token (exact
    or a reported near-tie). Returns the worst hidden-state error."""
    L = m["n_layers"]
    moe = m["n_experts"] > 0
    worst = 0.0
    for l in (range(L) if layers is None else layers):
        if moe and ids is not None:
            g_ids = [int(v) for v in ids[l, b].cpu().tolist()]
            o_ids = [int(v) for v in ref["topk_ids"][rb][l]]
            assert g_ids == o_ids, f"sequence {b} layer {l}: top-k {g_ids} != oracle {o_ids}"
            if tw is not None:
                assert rel_err(tw[l, b], ref["topk_w"][rb][l]) < 1e-3
            assert rel_err(dec.router_logits(l)[b], ref["router_logits"][rb][l]) < HIDDEN_TOL
        e_a = rel_err(dec.hidden_after_attn(l)[b], ref["x_attn"][rb][l])
        e_f = rel_err(dec.hidden_after_ffn(l)[b], ref["x_ffn"][rb][l])
        assert e_a < HIDDEN_TOL, f"sequence {b} layer {l}: attention residual rel err {e_a}"
        assert e_f < HIDDEN_TOL, f"sequence {b} layer {l}: FFN residual rel err {e_f}"
        assert max(e_a, e_f) < REGRESSION_TOL, f"sequence {b} layer {l}: accuracy regression ({e_a}, {e_f})"
        worst = max(worst, e_a, e_f)
        if pool_slot is not None:
            for g in range(m["n_kv_heads"]):
                k, v = pool_slot(dec, m, b, l, g, pos)
                assert rel_err(k.float(), ref["k_new"][rb][l][g].float()) < HIDDEN_TOL
                assert rel_err(v.float(), ref["v_new"][rb][l][g].float()) < HIDDEN_TOL
    if logits is not None:
        e_l = rel_err(logits[b], ref["logits"][rb])
        assert e_l < HIDDEN_TOL, f"sequence {b}: logits rel err {e_l}"
        assert e_l < REGRESSION_TOL, f"sequence {b}: logits accuracy regression ({e_l})"
        worst = max(worst, e_l)
    if tok_out is not None:
        got, want = int(tok_out[b]), ref["next"][rb]
        if got != want:
            assert argmax_near_tie(ref["logits"][rb], got, want), f"sequence {b}: next {got} != {want}"
            flush(f"  sequence {b}: near-tie in argmax: {got} vs {want}")
    return worst
