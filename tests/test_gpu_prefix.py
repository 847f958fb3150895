"""GPU decode over a shared prefix, through the C ABI.

A finished request A (700 tokens) is frozen as a checkpoint in the pool.
Two new requests lease with prefix sharing: B reuses 500 tokens of A and C
333, so each shares A's whole pages inside its match (the same physical
pages in both rows of the page table) and gets a private copy of the page
its match ends inside, copied on the device. Their own prior tokens past the
match are then filled with their own seeded KV (standing in for prefill)
and the batch decodes 4 steps. Each step is compared with the oracle on
contiguous KV spliced the same way (A's K/V below the match, the
sequence's own above): top-k ids, every layer's hidden state, the new K/V,
logits and the next token; and A's shared pages stay bit-identical, since
no one writes them.
"""
import pytest
import torch

import decode_megakernel_persistent_amd as mk
import oracle as O
from decode_megakernel_persistent_amd.runtime import Decoder, alloc_kv_pool, copy_kv_page
from fixtures import HostKV
from fixtures import device as fxd
from fixtures.hostmodel import HostWeights
from fixtures.session import spec
from gpu_util import NEAR_TIE, compare_sequence, flush, gpu_routing
from test_gpu_step import _pool_slot

pytestmark = pytest.mark.gpu


class Spliced:
    """Prior KV of batch row b: the checkpoint's (fixture sequence 0) below
    cut[b], the row's own (fixture sequence own[b]) from there on."""

    def __init__(self, kv, cut, own):
        self.kv, self.cut, self.own = kv, cut, own

    def _get(self, f, l, b, g, c):
        a, o = f(l, 0, g, c), f(l, self.own[b], g, c)
        return torch.cat([a[:self.cut[b]], o[self.cut[b]:]])

    def k(self, l, b, g, c):
        return self._get(self.kv.k, l, b, g, c)

    def v(self, l, b, g, c):
        return self._get(self.kv.v, l, b, g, c)


def test_decode_over_shared_checkpoint_pages():
    seed, steps = 0, 4
    m = spec("small_moe", seed)["model"]
    L, V, pt = m["n_layers"], m["vocab"], m["page_tokens"]
    K = m["top_k"]
    n_pages = 400
    g = torch.Generator().manual_seed(11)
    A = torch.randint(0, V, (700,), generator=g).tolist()
    pool = mk.mk_pool_create(n_pages, pt, 4, list(range(n_pages)))
    kvpool = alloc_kv_pool(m, n_pages, "cuda")
    mk.mk_pool_lease_prefix(pool, 100, A, len(A))
    row_a = torch.tensor(mk.mk_pool_page_table(pool, [100], -(-len(A) // pt))[0], dtype=torch.int32, device="cuda")
    fxd.fill_kv(kvpool, row_a, m, seed, 0, len(A))
    mk.mk_pool_finish(pool, 100, A)
    a_pages = row_a.cpu().tolist()
    flush(f"[prefix] checkpoint of {len(A)} tokens on pages {a_pages[0]}..{a_pages[-1]}")

    cuts, prompts = [500, 333], []
    for b, cut in enumerate(cuts):
        tail = torch.randint(0, V, (41 + 50 * b,), generator=g).tolist()
        tail[0] = (A[cut] + 1) % V                        # the prompts part from A right at the cut
        prompts.append(A[:cut] + tail)
    ctx = [len(p) - 1 for p in prompts]                   # prior tokens; the last prompt token runs
    copies = []
    for b, p in enumerate(prompts):
        slot, matched, src, dst = mk.mk_pool_lease_prefix(pool, b, p, len(p) + steps)
        assert matched == cuts[b] and slot == b
        assert (src, dst) != (-1, -1) and src == a_pages[cuts[b] // pt]
        copies.append((src, dst))
    max_pages = max(mk.mk_pool_seq_pages(pool, b) for b in range(2))
    rows = mk.mk_pool_page_table(pool, [0, 1], max_pages)
    for b in range(2):
        assert rows[b][:cuts[b] // pt] == a_pages[:cuts[b] // pt]        # shared, the same pages
    for src, dst in copies:
        copy_kv_page(m, kvpool, src, dst)
    row_dev = torch.tensor(rows, dtype=torch.int32, device="cuda")
    for b in range(2):
        fxd.fill_kv(kvpool, row_dev[b], m, seed, 1 + b, ctx[b], start=cuts[b])
    torch.cuda.synchronize()
    shared_before = {p: kvpool.view(-1, kvpool.numel() // n_pages)[p].clone() for p in a_pages}

    W = fxd.weights(m, seed, "cuda")
    bounds = [c + steps for c in ctx]
    dec = Decoder(m, W, kvpool, n_pages, ctx, rows, max_pages, max(bounds), ctx_bounds=bounds)
    Wh = HostWeights(m, seed)
    kv = O.OracleKV(m, ctx, steps, Spliced(HostKV(m, seed), cuts, [1, 2]))
    tok = torch.tensor([p[-1] for p in prompts], dtype=torch.int32, device="cuda")
    ids = torch.full((L, 2, K), -1, dtype=torch.int32, device="cuda")
    tw = torch.zeros((L, 2, K), dtype=torch.float32, device="cuda")
    logits = torch.zeros((2, V), dtype=torch.float32, device="cuda")
    worst = 0.0
    for s in range(steps):
        out = torch.full((2,), -1, dtype=torch.int32, device="cuda")
        dec.step(tok, out, ids, tw, logits)
        torch.cuda.synchronize()
        dec.check_status()
        ref, forced, differ = O.decode_step_following(m, Wh, kv, tok.cpu().tolist(),
                                                      [gpu_routing(ids, b) for b in range(2)], NEAR_TIE)
        assert not differ
        for b in range(2):
            worst = max(worst, compare_sequence(dec, m, b, ref, b, ids, tw, logits, out, ctx[b] + s, _pool_slot))
        tok = out
    for p, before in shared_before.items():
        assert torch.equal(kvpool.view(-1, kvpool.numel() // n_pages)[p].view(torch.int16),
                           before.view(torch.int16)), f"shared page {p} was written"
    flush(f"  {steps} steps over shared pages match the oracle (worst rel err {worst:.2e}); "
          f"{len(a_pages)} checkpoint pages untouched")
    mk.mk_pool_free(pool)
    dec.close()
