"""The folded router (batch-1 MoE) on the GPU.

- mk_router_fold: its first columns W_r diag(g) exactly, and the product
  W_r diag(g) W_o against fp64 from the host
  weights (each term is a product of three bf16 values, exact in fp32; the
  fp32 sums of H = 1024 terms carry a rounding walk of about sqrt(H) 2^-24,
  2e-6 of the result's scale, so 1e-5 is the bar), with non-unit gains so
  that the diagonal is exercised;
- the unfolded router stage (MK_PLAN_NO_ROUTER_FOLD) still matches the
  oracle on a whole small-MoE step (every other batch-1 MoE case runs folded).
"""
import pytest
import torch

import decode_megakernel_persistent_amd as mk
from fixtures import device as fxd
from fixtures.hostmodel import HostWeights
from fixtures.session import spec
from test_gpu_step import run_step_parity

pytestmark = pytest.mark.gpu


def test_fold_equals_the_fp64_product():
    m = spec("small_moe", 0)["model"]
    L, E, H, K = m["n_layers"], m["n_experts"], m["hidden"], m["n_q_heads"] * m["head_dim"]
    W = fxd.weights(m, 0, "cuda")
    g = torch.Generator().manual_seed(3)
    gains = (0.5 + torch.rand((L, H), generator=g)).to(torch.bfloat16)
    W["ffn_norm"] = gains.cuda()
    out = torch.empty((L, E, H + K), dtype=torch.float32, device="cuda")
    w = mk.mk_weights(*[W[k].data_ptr() if W.get(k) is not None else None for k, _ in mk.mk_weights._fields_])
    mk.mk_router_fold(mk.model_desc(m), w, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    Hw = HostWeights(m, 0)
    for l in range(L):
        rg = Hw.router(l).double() * gains[l].double()[None, :]
        got = out[l].cpu().double()
        assert torch.equal(got[:, :H], rg), f"layer {l}: W_r diag(g) is not exact"
        want = rg @ Hw.wo(l).double()
        err = ((got[:, H:] - want).abs().max() / want.abs().max()).item()
        assert err < 1e-5, f"layer {l}: fold rel err {err}"


def test_unfolded_router_stage_step():
    run_step_parity("small_moe", plan_flags=mk.MK_PLAN_NO_ROUTER_FOLD)
