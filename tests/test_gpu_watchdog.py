"""The step's deadline, forced from the host, and recovery from it.

The device image of a plan is edited on the host before upload: one task's
op is cleared, so the outputs it produces (the attention residual rows of a
tile of the middle layer) are never written in that step and every task that
needs them waits. The kernel's own bounded wait must then record
MK_ETIMEOUT, naming a task at or after that layer, and every workgroup must
leave: the step ends within a short multiple of the deadline, the greedy
token is not written and no sequence length advances. Then the good image
goes back, the decoder recovers (status and counters zeroed, lengths put
back) and the next step, with a new epoch, matches the oracle layer by
layer, with its counters at exactly one step's count.
"""
import time

import numpy as np
import pytest
import torch

import oracle as O
from fixtures.session import gpu_session, oracle_inputs, spec
from fixtures.hostmodel import DeviceCopyWeights
from gpu_util import NEAR_TIE, check_counters_against_oracle, compare_sequence, flush, gpu_routing, plan_bounds
from test_gpu_step import _pool_slot
from test_lib_cpu import OP_BO, OP_O, decode_plan

pytestmark = pytest.mark.gpu


def upload(dec, img):
    dec.plan_buf.copy_(torch.frombuffer(bytearray(img), dtype=torch.uint8))
    torch.cuda.synchronize()


def run_watchdog(name, deadline_ms, weights_from_device=False, **over):
    import decode_megakernel_persistent_amd as mk
    w = spec(name, 0, **over)
    m, B = w["model"], w["batch"]
    L, V = m["n_layers"], m["vocab"]
    K = m["top_k"] if m["n_experts"] else 1
    dec, pool, Wd = gpu_session(w, 0)
    dev = dec.device
    good = mk.mk_plan_export(dec.plan)
    _, _, _, tasks = decode_plan(good)
    layer = L // 2
    picks = np.nonzero(((tasks["op"] == OP_O) | (tasks["op"] == OP_BO)) & (tasks["layer"] == layer))[0]
    drop = int(picks[len(picks) // 2])
    bad = bytearray(good)
    off = int(np.frombuffer(good, dtype="<u4", count=16)[4]) + drop * tasks.dtype.itemsize
    bad[off] = 0          # op: none
    bad[off + 1] = 0      # flags
    flush(f"[watchdog] {name}: task {drop} (O projection of layer {layer}) removed; deadline {deadline_ms} ms")
    upload(dec, bytes(bad))
    tok_in = torch.tensor(w["tokens"], dtype=torch.int32, device=dev)
    tok_out = torch.full((B,), -1, dtype=torch.int32, device=dev)
    lens0 = list(w["ctx"])
    t0 = time.perf_counter()
    dec.step(tok_in, tok_out, timeout_ms=deadline_ms)
    torch.cuda.synchronize()
    took = time.perf_counter() - t0
    with pytest.raises(mk.MkError) as e:
        dec.check_status()
    st = dec.status.cpu().tolist()
    flush(f"  step ended after {took * 1e3:.1f} ms: {e.value}")
    assert e.value.status == mk.MK_ETIMEOUT
    ti = st[1] & 0xFFFFFFFF
    assert ti < len(tasks) and ti != drop
    assert int(tasks["layer"][ti]) >= layer, f"timed out in task {ti} of layer {int(tasks['layer'][ti])}"
    assert took < 20 * deadline_ms / 1e3 + 2.0
    assert tok_out.cpu().tolist() == [-1] * B
    assert dec.seq_lens.cpu().tolist() == lens0

    # recovery: the good image, a new epoch, one step matching the oracle
    upload(dec, good)
    dec.recover(lens0)
    ids = torch.full((L, B, K), -1, dtype=torch.int32, device=dev)
    tw = torch.zeros((L, B, K), dtype=torch.float32, device=dev)
    logits = torch.zeros((B, V), dtype=torch.float32, device=dev)
    dec.step(tok_in, tok_out, ids, tw, logits)
    torch.cuda.synchronize()
    dec.check_status()
    assert dec.seq_lens.cpu().tolist() == [c + 1 for c in lens0]
    if weights_from_device:
        Wh = DeviceCopyWeights(m, Wd, 0)
        _, kv = oracle_inputs(w, 0, cache=False)
    else:
        Wh, kv = oracle_inputs(w, 0)
    ref, forced, differ = O.decode_step_following(m, Wh, kv, w["tokens"],
                                                  [gpu_routing(ids, b) for b in range(B)] if m["n_experts"] else None,
                                                  NEAR_TIE)
    assert not differ
    worst = max(compare_sequence(dec, m, b, ref, b, ids if m["n_experts"] else None, tw, logits, tok_out, lens0[b],
                                 _pool_slot) for b in range(B))
    exp = O.expected_counters(m, plan_bounds(w))
    check_counters_against_oracle(mk.mk_plan_counter_names(dec.plan), dec.counters().tolist(), exp, steps=1)
    flush(f"  recovered: epoch {dec.epoch} step matches the oracle (worst rel err {worst:.2e})")
    mk.mk_pool_free(pool)
    dec.close()


def test_small_moe_deadline_then_recovery():
    run_watchdog("small_moe", 20)


def test_batch_deadline_then_recovery():
    run_watchdog("small_moe_b5", 20)


def test_moe48_8k_deadline_then_recovery():
    run_watchdog("moe48_b1_8k", 50, weights_from_device=True)
