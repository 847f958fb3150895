"""GPU decode across plan refreshes (mk_plan_update), through the C ABI.

Pages are leased as the sequences grow, not for the worst case up front:
each sequence holds exactly the pages its next token needs, the pool maps a
new page when a sequence reaches a page boundary, and before every step the
plan is refreshed with the new lengths, page table and the tightest bounds
(length + 1). Each step is compared with the oracle, teacher-forced on the
GPU's input tokens and following its routing at near-ties: top-k ids, every
layer's hidden state, the new K and V in the pool, logits and the next token;
and after each step the completion counters against the oracle's counts for
that step's bounds, times the steps since the last restart. Cases: a batch of
five ragged sequences (two cross a page boundary in the first step), one
sequence crossing a boundary mid-run, and the attention split queue, whose
item count changes with the bound (the planner then asks for a restart).
"""
import pytest
import torch

import oracle as O
from fixtures import device as fxd
from fixtures.session import oracle_inputs, page_order, spec
from gpu_util import NEAR_TIE, check_counters_against_oracle, compare_sequence, flush, gpu_routing
from test_gpu_step import _pool_slot

pytestmark = pytest.mark.gpu


def run_growing(name, n_steps, seed=0, plan_flags=0, **over):
    import decode_megakernel_persistent_amd as mk
    from decode_megakernel_persistent_amd.runtime import Decoder, alloc_kv_pool
    w = spec(name, seed, steps=n_steps, **over)
    m, B = w["model"], w["batch"]
    L, V, pt = m["n_layers"], m["vocab"], m["page_tokens"]
    moe = m["n_experts"] > 0
    K = m["top_k"] if moe else 1
    flush(f"[plan update] {name} ctx={w['ctx']} steps={n_steps} flags={plan_flags}")
    pool = mk.mk_pool_create(w["pool_pages"], pt, B, [int(v) for v in page_order(w, seed)])
    lens = list(w["ctx"])
    for b in range(B):
        mk.mk_pool_lease(pool, b, lens[b] + 1)
    max_pages = max(-(-(c + n_steps) // pt) for c in lens)
    rows = mk.mk_pool_page_table(pool, list(range(B)), max_pages)
    kvpool = alloc_kv_pool(m, w["pool_pages"], "cuda")
    Wd = fxd.weights(m, seed, "cuda")

    def bounds():
        cb = [c + 1 for c in lens]
        return max(cb), (cb if B > 1 else None)

    bound, cb = bounds()
    dec = Decoder(m, Wd, kvpool, w["pool_pages"], lens, rows, max_pages, bound, plan_flags=plan_flags,
                  ctx_bounds=cb)
    for b in range(B):
        fxd.fill_kv(kvpool, dec.page_table[b], m, seed, b, lens[b])
    torch.cuda.synchronize()
    Wh, kv = oracle_inputs(w, seed)
    dev = dec.device
    tok = torch.tensor(w["tokens"], dtype=torch.int32, device=dev)
    ids = torch.full((L, B, K), -1, dtype=torch.int32, device=dev)
    tw = torch.zeros((L, B, K), dtype=torch.float32, device=dev)
    logits = torch.zeros((B, V), dtype=torch.float32, device=dev)
    restarts = images = 0
    worst = 0.0
    for s in range(n_steps):
        out = torch.full((B,), -1, dtype=torch.int32, device=dev)
        dec.step(tok, out, ids, tw, logits)
        torch.cuda.synchronize()
        dec.check_status()
        assert dec.seq_lens.cpu().tolist() == [c + 1 for c in lens]
        tokens = tok.cpu().tolist()
        ref, forced, differ = O.decode_step_following(m, Wh, kv, tokens,
                                                      [gpu_routing(ids, b) for b in range(B)] if moe else None,
                                                      NEAR_TIE)
        assert not differ, f"step {s}: top-k differs from the oracle without a near-tie at {differ}"
        for b in range(B):
            worst = max(worst, compare_sequence(dec, m, b, ref, b, ids if moe else None, tw, logits, out,
                                                lens[b], _pool_slot))
        exp = O.expected_counters(m, cb if cb is not None else [bound])
        check_counters_against_oracle(mk.mk_plan_counter_names(dec.plan), dec.counters().tolist(), exp,
                                      steps=dec.epoch)
        # the next step: one more token per sequence, a page where it needs one
        lens = [c + 1 for c in lens]
        for b in range(B):
            mk.mk_pool_extend(pool, b, lens[b] + 1)
        rows = mk.mk_pool_page_table(pool, list(range(B)), max_pages)
        bound, cb = bounds()
        ch = dec.update(lens, rows, bound, cb)
        images += bool(ch & mk.MK_PLAN_CHANGED_IMAGE)
        restarts += bool(ch & (mk.MK_PLAN_CHANGED_WORKSPACE | mk.MK_PLAN_CHANGED_COUNTERS))
        tok = out
    flush(f"  {n_steps} steps: image re-uploaded {images} times, restarted {restarts} times; "
          f"worst rel err {worst:.2e}")
    assert [mk.mk_pool_seq_pages(pool, b) for b in range(B)] == [-(-(c + 1) // pt) for c in lens]
    mk.mk_pool_free(pool)
    dec.close()
    return images, restarts


def test_batch_grows_through_page_boundaries():
    # contexts 2048, 1, 517, 1300, 16: sequences 0 and 4 need a new page at once
    images, restarts = run_growing("small_moe_b5", 20)
    assert images == 20 and restarts >= 2


def test_one_sequence_crosses_a_page():
    images, restarts = run_growing("small_moe", 12, ctx=[2040])
    assert restarts >= 1


def test_attention_queue_restarts_when_its_items_change():
    import decode_megakernel_persistent_amd as mk
    images, restarts = run_growing("tiny_dense", 40, ctx=[100], plan_flags=mk.MK_PLAN_ATTN_QUEUE)
    assert restarts >= 2
