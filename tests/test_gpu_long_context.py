"""GPU parity at long context (262144 prior tokens), through the C ABI.

- The small MoE with 262143 prior tokens (16385 pages, the last one partly
  filled): one full step against the oracle, as in test_gpu_step.
- The 48-layer MoE at its full long-context size (262144 prior tokens,
  about 25 GB of paged KV): one step in the launch configuration the
  benchmark times, checked on outputs the oracle computes one by one -- the
  queries, the new K and V in the pool and the attention output of layer 0
  (all 32 query heads over all 262145 positions) -- plus the properties
  that hold at any size: status, completion counters against the oracle's
  counts, sequence length, a token in the vocabulary.
"""
import pytest
import torch

import oracle as O
from fixtures.hostmodel import HostKV, HostWeights
from fixtures.session import gpu_session, spec
from gpu_util import HIDDEN_TOL, check_device_counters, flush, rel_err
from test_gpu_step import _pool_slot, run_step_parity

pytestmark = pytest.mark.gpu


def test_small_moe_long_context():
    run_step_parity("small_moe", ctx=[262143], pool_pages=16500)


def layer0_reference(m, seed, tok, pos, b=0):
    """Oracle pieces of layer 0 for sequence b at position pos: q [Hq][d]
    after rotation, bf16 k and v of the new token [Hkv][d], attention output
    [Hq][d] over the pos prior tokens and the new one."""
    W = HostWeights(m, seed, cache=False)
    kv = HostKV(m, seed)
    H, Hq, Hkv, d = m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    x = W.embed_row(tok).to(torch.float32)
    u = O.rmsnorm(x, W.attn_norm(0), m["rms_eps"])
    y = O.matvec(W.wqkv(0), u)
    q = y[: Hq * d].view(Hq, d)
    k = y[Hq * d:(Hq + Hkv) * d].view(Hkv, d)
    v = y[(Hq + Hkv) * d:].view(Hkv, d)
    cos, sin = O.rope_cos_sin(m["rope_theta"], d, pos)
    q = O.rope(q, cos, sin)
    k_new = O.to_bf16(O.rope(k, cos, sin))
    v_new = O.to_bf16(v)
    hg = Hq // Hkv
    out = torch.empty(Hq, d, dtype=torch.float32)
    for g in range(Hkv):
        K = torch.cat([kv.k(0, b, g, pos), k_new[g:g + 1]])
        V = torch.cat([kv.v(0, b, g, pos), v_new[g:g + 1]])
        out[g * hg:(g + 1) * hg] = O.attention(q[g * hg:(g + 1) * hg], K, V)
    return q, k_new, v_new, out


def test_moe48_262144_layer0_sampled():
    w = spec("moe48_b1_256k", 0)
    m = w["model"]
    pos = w["ctx"][0]
    flush(f"[long context] moe48_b1_256k ctx={pos}: setting up weights and KV on the device")
    dec, pool, _ = gpu_session(w, 0)
    dev = dec.device
    tok_in = torch.tensor(w["tokens"], dtype=torch.int32, device=dev)
    tok_out = torch.full((1,), -1, dtype=torch.int32, device=dev)
    flush("  one step")
    dec.step(tok_in, tok_out)
    torch.cuda.synchronize()
    dec.check_status()
    assert 0 <= int(tok_out[0]) < m["vocab"]
    assert dec.seq_lens.cpu().tolist() == [pos + 1]
    import decode_megakernel_persistent_amd as mk
    check_device_counters(dec, w)

    flush("  oracle: layer 0 at full context")
    q_ref, k_ref, v_ref, o_ref = layer0_reference(m, 0, w["tokens"][0], pos)
    e_q = rel_err(dec.queries(0)[0], q_ref)
    e_o = rel_err(dec.attn_out(0)[0], o_ref)
    flush(f"  layer 0: query rel err {e_q:.2e}, attention output rel err {e_o:.2e}")
    assert e_q < HIDDEN_TOL and e_o < HIDDEN_TOL
    for g in range(m["n_kv_heads"]):
        k, v = _pool_slot(dec, m, 0, 0, g, pos)
        assert rel_err(k.float(), k_ref[g].float()) < HIDDEN_TOL
        assert rel_err(v.float(), v_ref[g].float()) < HIDDEN_TOL
    mk.mk_pool_free(pool)
    dec.close()
