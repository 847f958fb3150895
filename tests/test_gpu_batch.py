"""GPU parity of batch decode steps (several sequences per step) against the oracle.

A batch plan runs the dense projections as MFMA tiles over all sequences, a
router/top-k task per sequence and expert tasks shared by the sequences
routed to them; each expert task takes an equal share of the rows of the
experts the routing chose (one case keeps a fixed expert part per task). Each case compares every sequence of one step with the
oracle exactly as the batch-1 cases do (greedy token, logits, hidden state
after every residual, new K/V in the pool, top-k ids, counters), on ragged
contexts that include an empty one and a single token. Six more cases draw
their shape (model, batch, contexts, steps ahead, unit count, attention
queue) from a seeded generator.
"""
import pytest

from test_gpu_step import greedy_agreement, run_step_parity

pytestmark = pytest.mark.gpu


def test_tiny_dense_batch3():
    # contexts 128, 0, 47: a full page set, an empty cache and a ragged tail
    run_step_parity("tiny_dense_b3")


def test_small_moe_batch5():
    # contexts 2048, 1, 517, 1300, 16
    run_step_parity("small_moe_b5")


def test_small_moe_batch32_ragged():
    # 32 sequences, contexts uniform in [1, 1024]: both MFMA column blocks
    run_step_parity("small_moe_b32")


def test_small_moe_batch5_greedy_16():
    greedy_agreement("small_moe_b5", 16)


def test_small_moe_batch5_fixed_expert_parts():
    # every expert task on one fixed (expert, part), not shares of the
    # experts the routing chose
    import decode_megakernel_persistent_amd as mk
    run_step_parity("small_moe_b5", plan_flags=mk.MK_PLAN_NO_EXPERT_SHARE)


def test_batch_attention_split_queue():
    # the batch's attention splits pulled from one shared queue (longest
    # first, from the plan's split table) instead of dealt to fixed units
    import decode_megakernel_persistent_amd as mk
    run_step_parity("small_moe_b5", plan_flags=mk.MK_PLAN_ATTN_QUEUE)
    run_step_parity("small_moe_b32", plan_flags=mk.MK_PLAN_ATTN_QUEUE)


def random_shapes(n, seed=7):
    """n seeded step shapes around the two small models that the planner
    accepts: batch 1 to 12, ragged contexts (some empty), 1 to 40 steps
    ahead, 64 to 256 units, with and without the attention queue."""
    import random
    import decode_megakernel_persistent_amd as mk
    from fixtures.session import lease_pages, spec
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        base = rng.choice(["tiny_dense", "small_moe"])
        B = 1 if rng.random() < 0.3 else rng.randint(2, 12)
        hi = 600 if base == "tiny_dense" else 1200
        ctx = [rng.choice([0, 1, rng.randint(0, hi)]) if rng.random() < 0.2 else rng.randint(0, hi)
               for _ in range(B)]
        steps = rng.randint(1, 40)
        n_cu = rng.randint(64, 256)
        flags = mk.MK_PLAN_ATTN_QUEUE if rng.random() < 0.4 else 0
        w = spec(base, 0, batch=B, ctx=ctx, steps=steps, pool_pages="sum*1.1")
        pool, rows, max_pages = lease_pages(w, 0)
        try:
            cb = [c + steps for c in w["ctx"]] if B > 1 else None
            p = mk.mk_plan(mk.model_desc(w["model"]), w["ctx"], [v for r in rows for v in r], max_pages,
                           max(w["ctx"]) + steps, n_cu=n_cu, flags=flags, ctx_bounds=cb)
            mk.mk_plan_free(p)
        except mk.MkError:
            continue  # a shape the library refuses (checked on the CPU)
        finally:
            mk.mk_pool_free(pool)
        out.append((base, dict(batch=B, ctx=ctx, steps=steps, pool_pages="sum*1.1"), n_cu, flags))
    return out


@pytest.mark.parametrize("case", range(6))
def test_random_shape_step_parity(case):
    # one step of a seeded random shape (see random_shapes) against the
    # oracle, every sequence as in the named cases above
    base, over, n_cu, flags = random_shapes(6)[case]
    run_step_parity(base, plan_flags=flags, n_cu=n_cu, **over)
