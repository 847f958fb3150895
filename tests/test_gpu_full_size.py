"""GPU parity of the 48-layer MoE at its measured sizes, through the C ABI,
in the launch configuration the benchmark times (one persistent launch over
every compute unit): batch 1 at 8192 prior tokens, and batch 32 with ragged
contexts of 512 to 32768 tokens. The whole step is too large for the oracle,
so layer 0 is checked on outputs the oracle computes one by one -- the
rotated queries, the new K and V in the pool, the attention output, the
hidden state after the O projection and residual, the router logits and the
top-k ids (bit-exact, or a reported near-tie) -- for the one sequence at
batch 1 and for three sampled sequences at batch 32 (the first, the longest
and the shortest context), plus the properties that hold at any size:
status, counters at epoch x producers, sequence lengths, next tokens in the
vocabulary.
"""
import pytest
import torch

import oracle as O
from fixtures.hostmodel import HostWeights
from fixtures.session import gpu_session, spec
from gpu_util import HIDDEN_TOL, flush, rel_err, topk_near_tie
from test_gpu_long_context import layer0_reference
from test_gpu_step import _pool_slot

pytestmark = pytest.mark.gpu


def layer0_ffn_input(m, seed, tok, o_ref):
    """Oracle: hidden state after layer 0's attention residual, and the
    router logits of that hidden state (empty for a dense FFN)."""
    W = HostWeights(m, seed, cache=False)
    x = W.embed_row(tok).to(torch.float32)
    xa = x + O.matvec(W.wo(0), o_ref.reshape(-1))
    if not m["n_experts"]:
        return xa, None
    u = O.rmsnorm(xa, W.ffn_norm(0), m["rms_eps"])
    return xa, O.matvec(W.router(0), u)


def check_sequence(dec, m, seed, b, tok, pos, topk_ids):
    q_ref, k_ref, v_ref, o_ref = layer0_reference(m, seed, tok, pos, b)
    e_q = rel_err(dec.queries(0)[b], q_ref)
    e_o = rel_err(dec.attn_out(0)[b], o_ref)
    for g in range(m["n_kv_heads"]):
        k, v = _pool_slot(dec, m, b, 0, g, pos)
        assert rel_err(k.float(), k_ref[g].float()) < HIDDEN_TOL
        assert rel_err(v.float(), v_ref[g].float()) < HIDDEN_TOL
    xa_ref, r_ref = layer0_ffn_input(m, seed, tok, o_ref)
    e_x = rel_err(dec.hidden_after_attn(0)[b], xa_ref)
    e_r = rel_err(dec.router_logits(0)[b], r_ref)
    flush(f"  sequence {b} (context {pos}): layer 0 query {e_q:.2e}, attention {e_o:.2e}, "
          f"hidden {e_x:.2e}, router {e_r:.2e}")
    assert max(e_q, e_o, e_x, e_r) < HIDDEN_TOL
    K = m["top_k"]
    g_ids = topk_ids[0, b].tolist()
    o_ids = O.topk(O.softmax(r_ref), K).tolist()
    if g_ids != o_ids:
        assert topk_near_tie(r_ref, K), f"top-k {g_ids} != oracle {o_ids} without a near-tie"
        flush(f"  near-tie in top-k: {g_ids} vs {o_ids}")


def run_full_size(name, sample):
    w = spec(name, 0)
    m, B = w["model"], w["batch"]
    flush(f"[full size] {name}: batch {B}, contexts {min(w['ctx'])}..{max(w['ctx'])}: "
          f"setting up weights and KV on the device")
    dec, pool, _ = gpu_session(w, 0)
    dev = dec.device
    tok_in = torch.tensor(w["tokens"], dtype=torch.int32, device=dev)
    tok_out = torch.full((B,), -1, dtype=torch.int32, device=dev)
    ids = torch.full((m["n_layers"], B, m["top_k"]), -1, dtype=torch.int32, device=dev)
    flush("  one step")
    dec.step(tok_in, tok_out, topk_ids=ids)
    torch.cuda.synchronize()
    dec.check_status()
    nxt = tok_out.cpu()
    assert bool(((nxt >= 0) & (nxt < m["vocab"])).all())
    assert dec.seq_lens.cpu().tolist() == [c + 1 for c in w["ctx"]]
    import decode_megakernel_persistent_amd as mk
    tg = torch.tensor(mk.mk_plan_counter_targets(dec.plan), dtype=torch.int64)
    assert torch.equal(dec.counters(), tg * dec.epoch)
    ids = ids.cpu()
    for b in sample(w["ctx"]):
        check_sequence(dec, m, 0, b, w["tokens"][b], w["ctx"][b], ids)
    mk.mk_pool_free(pool)
    dec.close()


def test_moe48_8k_layer0_sampled():
    run_full_size("moe48_b1_8k", lambda ctx: [0])


def test_moe48_batch32_ragged_layer0_sampled():
    def pick(ctx):
        longest = max(range(len(ctx)), key=lambda b: ctx[b])
        shortest = min(range(len(ctx)), key=lambda b: ctx[b])
        return sorted({0, longest, shortest})
    run_full_size("moe48_b32_ragged", pick)
