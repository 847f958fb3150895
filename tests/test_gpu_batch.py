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


def test_small_moe_batch5_row_major_experts():
    # the expert GEMMs on the row-major gate, up and down rows (no tile copy)
    run_step_parity("small_moe_b5", expert_tiles=False)


@pytest.mark.parametrize("name", ["small_moe", "tiny_dense"])
def test_expert_tile_order(name):
    # mk_expert_tile against the tile order written out with tensor reshapes:
    # per layer and expert, gate/up rows interleaved then the down rows, in
    # 16-row blocks of 32-column k-steps, entry t = row t % 16, columns
    # 8 (t / 16) .. + 7; bit-exact
    import torch
    import decode_megakernel_persistent_amd as mk
    from fixtures import device as fxd
    from fixtures.session import spec
    m = spec(name, 0)["model"]
    W = fxd.weights(m, 0, "cuda")
    moe = m["n_experts"] > 0
    L, H = m["n_layers"], m["hidden"]
    E = m["n_experts"] if moe else 1
    F = m["expert_ffn"] if moe else m["ffn_dim"]
    out = torch.empty(L * E * 3 * F * H, dtype=torch.bfloat16, device="cuda")
    w0 = mk.mk_weights(*[None if W.get(k) is None else W[k].data_ptr() for k, _ in mk.mk_weights._fields_])
    mk.mk_expert_tile(mk.model_desc(m), w0, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    g = W["gate"].view(L, E, F, H).cpu().view(torch.int16)
    u = W["up"].view(L, E, F, H).cpu().view(torch.int16)
    d = W["down"].view(L, E, H, F).cpu().view(torch.int16)
    gu = torch.stack([g, u], dim=3).reshape(L, E, 2 * F, H)

    def tiles(x, R, K):
        # [L][E][R][K] -> [L][E][R/16][K/32][kq][r16][8]
        t = x.reshape(L, E, R // 16, 16, K // 32, 4, 8).permute(0, 1, 2, 4, 5, 3, 6)
        return t.reshape(L, E, R * K)
    want = torch.cat([tiles(gu, 2 * F, H), tiles(d, H, F)], dim=2).reshape(-1)
    assert torch.equal(out.cpu().view(torch.int16), want)


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
