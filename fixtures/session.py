"""Ready-to-step decode sessions on seeded synthetic inputs, and their oracle twins.

Test and benchmark infrastructure. `gpu_session` leases pages from the
library's host pool (seeded physical order), fills the device KV pool and
weights from the fixture generator and plans the batch; `oracle_inputs`
builds the matching host-side weights and contiguous KV for the oracle.
Neither computes any part of the decode step.
"""
import torch

from . import host
from .hostmodel import HostWeights, HostKV
from .workloads import resolve, workload


def spec(name, seed=0, **over):
    """Resolved workload: model, batch, ctx, steps, pool_pages, tokens."""
    return resolve(workload(name, **over), seed)


def page_order(w, seed=0):
    return host.permutation(seed, w["pool_pages"])


def lease_pages(w, seed=0):
    """(pool handle, page table rows, max_pages) from the library's host pool.

    Every sequence leases its worst case, ctx + steps tokens, all or nothing.
    """
    import decode_megakernel_persistent_amd as mk
    m, B = w["model"], w["batch"]
    pt = m["page_tokens"]
    pool = mk.mk_pool_create(w["pool_pages"], pt, B, [int(v) for v in page_order(w, seed)])
    for b in range(B):
        mk.mk_pool_lease(pool, b, w["ctx"][b] + w["steps"])
    max_pages = max((c + w["steps"] + pt - 1) // pt for c in w["ctx"])
    rows = mk.mk_pool_page_table(pool, list(range(B)), max_pages)
    return pool, rows, max_pages


def gpu_session(w, seed=0, device="cuda", weights=None, n_cu=0, attn_split_pages=0, trace=False,
                plan_flags=0, expert_tiles=True):
    """A Decoder for workload w with its KV filled; returns (decoder, pool handle, weights)."""
    import decode_megakernel_persistent_amd as mk
    from decode_megakernel_persistent_amd.runtime import Decoder, alloc_kv_pool
    from . import device as fxd
    m, B = w["model"], w["batch"]
    pool, rows, max_pages = lease_pages(w, seed)
    kvpool = alloc_kv_pool(m, w["pool_pages"], device)
    W = weights if weights is not None else fxd.weights(m, seed, device)
    bound = max(w["ctx"]) + w["steps"]
    ctx_bounds = [c + w["steps"] for c in w["ctx"]] if B > 1 else None
    dec = Decoder(m, W, kvpool, w["pool_pages"], w["ctx"], rows, max_pages, bound,
                  n_cu=n_cu, attn_split_pages=attn_split_pages, device=device, trace=trace,
                  plan_flags=plan_flags, ctx_bounds=ctx_bounds,
                  **({} if expert_tiles else {"expert_tiles": False}))
    for b in range(B):
        fxd.fill_kv(kvpool, dec.page_table[b], m, seed, b, w["ctx"][b])
    torch.cuda.synchronize(device)
    return dec, pool, W


def oracle_inputs(w, seed=0, cache=True):
    """(HostWeights, OracleKV) matching gpu_session(w, seed)."""
    import oracle as O
    m = w["model"]
    W = HostWeights(m, seed, cache=cache)
    kv = O.OracleKV(m, w["ctx"], w["steps"], HostKV(m, seed))
    return W, kv
