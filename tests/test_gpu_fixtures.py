"""The device fill of the seeded inputs equals the host generator, bit for bit.

The oracle draws its inputs with the host generator (fixtures/fx_host.c, the
definition) or, at full size, copies them from the device tensors that the
device implementation (fixtures/fx_gpu.hip) filled. Both routes rely on the
two implementations agreeing exactly, which these cases check: every weight
tensor of the small MoE in full, sampled matrices and rows of every kind of
the 48-layer MoE, the norm gains, and prior KV written through a shuffled
page table in the pool's documented page layout.
"""
import pytest
import torch

from fixtures import HostKV, HostWeights
from fixtures import device as fxd
from fixtures.hostmodel import DeviceCopyWeights
from fixtures.session import gpu_session, spec
from gpu_util import flush, kv_offsets

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    return torch.equal(a.view(torch.int16).cpu(), b.view(torch.int16).cpu())


def check_weights(m, Wd, picks):
    H = HostWeights(m, 0, cache=False)
    C = DeviceCopyWeights(m, Wd, 0, cache=False)
    for name, args in picks:
        a, b = getattr(H, name)(*args), getattr(C, name)(*args)
        assert a.shape == b.shape and same_bits(a, b), f"{name}{args}: device fill differs"
    for k in ("attn_norm", "ffn_norm", "final_norm"):
        assert bool((Wd[k].float() == 1.0).all()), f"{k}: gains are not 1.0"


def test_small_moe_weights_in_full():
    m = spec("small_moe", 0)["model"]
    Wd = fxd.weights(m, 0, "cuda")
    picks = [("embed_row", (t,)) for t in (0, 1, 31999)] + [("lm_head", ())]
    for l in range(m["n_layers"]):
        picks += [("wqkv", (l,)), ("wo", (l,)), ("router", (l,))]
        for e in range(m["n_experts"]):
            picks += [("gate", (l, e)), ("up", (l, e)), ("down", (l, e))]
    check_weights(m, Wd, picks)


def test_moe48_weights_sampled():
    m = spec("moe48_b1_8k", 0)["model"]
    flush("[fixtures] 48-layer weights on the device")
    Wd = fxd.weights(m, 0, "cuda")
    picks = [("embed_row", (t,)) for t in (0, 77777, 151935)] + [
        ("wqkv", (0,)), ("wqkv", (47,)), ("wo", (31,)), ("router", (0,)), ("router", (47,)),
        ("gate", (5, 100)), ("up", (12, 3)), ("down", (40, 127)), ("gate", (47, 0)), ("lm_head", ())]
    check_weights(m, Wd, picks)


@pytest.mark.parametrize("name,ctx", [("small_moe", [2048]), ("tiny_dense_b3", None)])
def test_prior_kv_through_the_page_table(name, ctx):
    over = {"ctx": ctx} if ctx else {}
    w = spec(name, 0, **over)
    m = w["model"]
    dec, pool, _ = gpu_session(w, 0)
    L, Hkv, d, pt = m["n_layers"], m["n_kv_heads"], m["head_dim"], m["page_tokens"]
    P = dec.pool.cpu().view(torch.int16)
    kv = HostKV(m, 0)
    koff = torch.stack([kv_offsets(sl, d)[0] for sl in range(pt)])   # [slot][dim]
    voff = torch.stack([kv_offsets(sl, d)[1] for sl in range(pt)])
    for b, c in enumerate(w["ctx"]):
        if c == 0:
            continue
        t = torch.arange(c)
        pages = dec.page_table[b].cpu().long()[t // pt]
        for l in range(L):
            for g in range(Hkv):
                base = ((pages * L + l) * Hkv + g) * 2 * pt * d
                got_k = P[base[:, None] + koff[t % pt]]
                got_v = P[base[:, None] + voff[t % pt]]
                assert torch.equal(got_k, kv.k(l, b, g, c).view(torch.int16)), f"K of sequence {b} layer {l} head {g}"
                assert torch.equal(got_v, kv.v(l, b, g, c).view(torch.int16)), f"V of sequence {b} layer {l} head {g}"
    import decode_megakernel_persistent_amd as mk
    mk.mk_pool_free(pool)
    dec.close()
