"""Workload shapes and the seeded synthetic-input recipe.

Shapes are the five decode workloads this repository measures and tests:
a tiny dense decoder, a small MoE, and a 48-layer MoE of ~30B total /
~3.3B active parameters at batch 1 / 8K context, at batch 32 with ragged
contexts, and at batch 1 / 262144 context. Input recipe (master seed 0):
weights N(0, 0.02) in bf16, RMSNorm gains 1.0, prior KV N(0, 1) in bf16,
first tokens uniform in [0, vocab), physical page order a seeded
permutation of the pool, ragged contexts uniform integers in [512, 32768].
"""
import copy

_MOE48 = dict(n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
              ffn_dim=0, n_experts=128, top_k=8, expert_ffn=768, norm_topk=1,
              vocab=151936, page_tokens=16, rms_eps=1e-6, rope_theta=1e4)

WORKLOADS = {
    "tiny_dense": dict(
        model=dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                   ffn_dim=512, n_experts=0, top_k=0, expert_ffn=0, norm_topk=1,
                   vocab=1024, page_tokens=16, rms_eps=1e-6, rope_theta=1e4),
        batch=1, ctx=[128], steps=256, pool_pages=64),
    "small_moe": dict(
        model=dict(n_layers=4, hidden=1024, n_q_heads=16, n_kv_heads=4, head_dim=64,
                   ffn_dim=0, n_experts=32, top_k=4, expert_ffn=512, norm_topk=1,
                   vocab=32000, page_tokens=16, rms_eps=1e-6, rope_theta=1e4),
        batch=1, ctx=[2048], steps=256, pool_pages=256),
    "moe48_b1_8k": dict(model=dict(_MOE48), batch=1, ctx=[8192], steps=256, pool_pages=1024),
    "moe48_b32_ragged": dict(model=dict(_MOE48), batch=32, ctx="uniform[512,32768]",
                             steps=256, pool_pages="sum*1.1"),
    "moe48_b1_256k": dict(model=dict(_MOE48), batch=1, ctx=[262144], steps=256,
                          pool_pages=16500),
    "moe48_b4_8k": dict(model=dict(_MOE48), batch=4, ctx=[8192, 8192, 8192, 8192], steps=256,
                        pool_pages="sum*1.1"),
}

# Batch parity cases on the small shapes: ragged contexts, one of them empty
# and one a single token, so that batch plans are checked against the oracle
# at sizes it finishes in seconds.
_TINY = WORKLOADS["tiny_dense"]["model"]
_SMALL = WORKLOADS["small_moe"]["model"]
WORKLOADS.update({
    "tiny_dense_b3": dict(model=dict(_TINY), batch=3, ctx=[128, 0, 47], steps=16, pool_pages=64),
    "small_moe_b5": dict(model=dict(_SMALL), batch=5, ctx=[2048, 1, 517, 1300, 16], steps=16,
                         pool_pages="sum*1.1"),
    "small_moe_b32": dict(model=dict(_SMALL), batch=32, ctx="uniform[1,1024]", steps=16,
                          pool_pages="sum*1.1"),
})

SIGMA_W = 0.02
SIGMA_KV = 1.0
NORM_GAIN_BITS = 0x3F80  # bf16 1.0


def workload(name, **over):
    w = copy.deepcopy(WORKLOADS[name])
    for k, v in over.items():
        if k in w["model"]:
            w["model"][k] = v
        else:
            w[k] = v
    return w


def resolve(w, seed=0):
    """Fill in drawn quantities: contexts, pool size, first tokens."""
    from . import host
    w = copy.deepcopy(w)
    m, B = w["model"], w["batch"]
    if isinstance(w["ctx"], str):
        lo, hi = (int(v) for v in w["ctx"][len("uniform["):-1].split(","))
        w["ctx"] = [int(v) for v in host.uniform(seed, host.FX_CTX, B, lo, hi)]
    pt = m["page_tokens"]
    if isinstance(w["pool_pages"], str):
        need = sum((c + w["steps"] + pt - 1) // pt for c in w["ctx"])
        w["pool_pages"] = int(need * 1.1) + 1
    w["tokens"] = [int(v) for v in host.uniform(seed, host.FX_TOKEN, B, 0, m["vocab"] - 1)]
    return w
