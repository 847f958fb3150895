"""The allocation-free step (mk_decode_step_static) against mk_decode_step.

Two decoders are set up on identical inputs (same weights, same pages, same
prior KV); one steps through mk_decode_step with its own workspace, the other
through mk_decode_step_static, whose workspace and counters live in the
library's static scratch. Every output must be bit-identical: greedy tokens,
top-k ids and weights, logits, sequence lengths and the whole KV pool. A
larger plan runs two steps first (the second on the scratch the first left,
with the next epoch), then a smaller plan two steps (the scratch is cleared
for the new plan and its epochs start again).
"""
import pytest
import torch

from fixtures.session import gpu_session, spec
from gpu_util import flush

pytestmark = pytest.mark.gpu


def run_pair(name, n_steps, **over):
    import decode_megakernel_persistent_amd as mk
    w = spec(name, 0, **over)
    m, B = w["model"], w["batch"]
    L, V = m["n_layers"], m["vocab"]
    K = m["top_k"] if m["n_experts"] else 1
    flush(f"[no-alloc] {name} ctx={w['ctx']} steps={n_steps}")
    ref, pool_r, Wd = gpu_session(w, 0)
    sta, pool_s, _ = gpu_session(w, 0, weights=Wd)
    dev = ref.device

    def bufs():
        return (torch.full((B,), -1, dtype=torch.int32, device=dev),
                torch.full((L, B, K), -1, dtype=torch.int32, device=dev),
                torch.zeros((L, B, K), dtype=torch.float32, device=dev),
                torch.zeros((B, V), dtype=torch.float32, device=dev))

    tok = torch.tensor(w["tokens"], dtype=torch.int32, device=dev)
    for s in range(n_steps):
        out_r, out_s = bufs(), bufs()
        ref.step(tok, *out_r)
        sta.step_static(tok, *out_s)
        torch.cuda.synchronize()
        ref.check_status()
        sta.check_status()
        for a, b, what in zip(out_r, out_s, ("tokens", "top-k ids", "top-k weights", "logits")):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"step {s}: {what} differ"
        assert torch.equal(ref.seq_lens, sta.seq_lens)
        assert torch.equal(ref.pool.view(torch.int16), sta.pool.view(torch.int16)), f"step {s}: KV pool differs"
        flush(f"  step {s}: next token {out_r[0].tolist()} identical through both entry points")
        tok = out_r[0]
    for d, p in ((ref, pool_r), (sta, pool_s)):
        mk.mk_pool_free(p)
        d.close()


def test_static_scratch_step_equals_the_caller_buffer_step():
    run_pair("small_moe", 2, ctx=[2048])
    run_pair("tiny_dense", 2, ctx=[100])
