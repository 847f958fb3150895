"""Shared helpers of the GPU parity tests (comparison metrics and triage)."""
import torch

# Hidden-state tolerance: max |gpu - oracle| / max |oracle| over a vector.
HIDDEN_TOL = 2e-2
# A top-k or argmax disagreement is a near-tie (reported, not failed) when
# the oracle's two competing scores differ by less than this fraction.
NEAR_TIE = 1e-5


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
