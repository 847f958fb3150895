"""GPU chunked prefill into the paged cache, through the C ABI.

A chunk of a sequence's prompt tokens runs as one step of the batch path
(MK_PLAN_PREFILL): its rows are consecutive positions of one sequence
sharing one page-table row, so MFMA tiles span the chunk and each row
attends to the prior context and to the chunk's earlier rows, whose K and V
are written into the shared pages in the same step. The oracle's definition
of a prefill is the decode step of each token in order. Compared per row:
top-k ids (bit-exact, following the GPU at near-ties), the hidden state
after every layer's attention and FFN residuals, the K and V written at the
row's position, the logits and the next token. Then a batch-1 plan decodes
on from the last row's token over the prefilled pages and is compared step
by step with the oracle continuing. Cases: a 20-token chunk crossing a page
boundary after 100 synthetic prior tokens, a full 32-token chunk from an
empty sequence, two chunks back to back, and a 16-token chunk of the
48-layer MoE after 8192 prior tokens.
"""
import pytest
import torch

import decode_megakernel_persistent_amd as mk
import oracle as O
from decode_megakernel_persistent_amd.runtime import Decoder, alloc_kv_pool
from fixtures import HostKV
from fixtures import device as fxd
from fixtures.hostmodel import DeviceCopyWeights, HostWeights
from fixtures.session import spec
from gpu_util import NEAR_TIE, compare_sequence, flush, gpu_routing
from test_gpu_step import _pool_slot

pytestmark = pytest.mark.gpu


def explain_difference(dec, m, b, ref, layer, ids):
    """Print how far row b's hidden states and router logits are from the
    oracle up to `layer`, and the oracle's top-k probability gap there."""
    from gpu_util import rel_err
    for l in range(layer + 1):
        ea = rel_err(dec.hidden_after_attn(l)[b], ref["x_attn"][0][l])
        ef = rel_err(dec.hidden_after_ffn(l)[b], ref["x_ffn"][0][l])
        er = rel_err(dec.router_logits(l)[b], ref["router_logits"][0][l])
        if l % 8 == 0 or l >= layer - 2:
            flush(f"    layer {l}: attn {ea:.2e} ffn {ef:.2e} router {er:.2e}")
    p = torch.softmax(ref["router_logits"][0][layer].double(), dim=-1)
    srt = torch.sort(p, descending=True).values
    k = m["top_k"]
    flush(f"    oracle top-k {ref['topk_ids'][0][layer].tolist()}, GPU {ids[layer, b].tolist()}; "
          f"p[k-1] {float(srt[k - 1]):.6e} p[k] {float(srt[k]):.6e} "
          f"gap {float((srt[k - 1] - srt[k]) / srt[k - 1]):.2e}")


def run_prefill(name, p0, chunks, n_decode, seed=0, weights_from_device=False):
    m = spec(name, seed)["model"]
    L, V, pt = m["n_layers"], m["vocab"], m["page_tokens"]
    K = m["top_k"] if m["n_experts"] else 1
    n_prompt = sum(chunks)
    total = p0 + n_prompt + n_decode
    n_pages = -(-total // pt) + 8
    pool = mk.mk_pool_create(n_pages, pt, 1, list(range(n_pages))[::-1])
    mk.mk_pool_lease(pool, 0, total)
    max_pages = -(-total // pt)
    row = mk.mk_pool_page_table(pool, [0], max_pages)[0]
    kvpool = alloc_kv_pool(m, n_pages, "cuda")
    W = fxd.weights(m, seed, "cuda")
    row_dev = torch.tensor(row, dtype=torch.int32, device="cuda")
    fxd.fill_kv(kvpool, row_dev, m, seed, 0, p0)
    torch.cuda.synchronize()
    Wh = DeviceCopyWeights(m, W, seed) if weights_from_device else HostWeights(m, seed)
    kv = O.OracleKV(m, [p0], n_prompt + n_decode, HostKV(m, seed))
    g = torch.Generator().manual_seed(7 + seed)
    prompt = torch.randint(0, V, (n_prompt,), generator=g).tolist()
    flush(f"[prefill] {name}: {p0} prior tokens, chunks {chunks}, then {n_decode} decode steps")
    pos, worst, nxt = p0, 0.0, None
    for C in chunks:
        toks = prompt[pos - p0: pos - p0 + C]
        lens = [pos + i for i in range(C)]
        dec = Decoder(m, W, kvpool, n_pages, lens, [row] * C, max_pages, pos + C,
                      plan_flags=mk.MK_PLAN_PREFILL, ctx_bounds=[x + 1 for x in lens])
        tok_in = torch.tensor(toks, dtype=torch.int32, device="cuda")
        out = torch.full((C,), -1, dtype=torch.int32, device="cuda")
        ids = torch.full((L, C, K), -1, dtype=torch.int32, device="cuda")
        tw = torch.zeros((L, C, K), dtype=torch.float32, device="cuda")
        logits = torch.zeros((C, V), dtype=torch.float32, device="cuda")
        dec.step(tok_in, out, ids if m["n_experts"] else None, tw if m["n_experts"] else None, logits)
        torch.cuda.synchronize()
        dec.check_status()
        for i, t in enumerate(toks):
            ref, forced, differ = O.decode_step_following(
                m, Wh, kv, [t], [gpu_routing(ids, i)] if m["n_experts"] else None, NEAR_TIE)
            if differ:
                explain_difference(dec, m, i, ref, differ[0][1], ids)
            assert not differ, f"row {i}: top-k differs without a near-tie at {differ}"
            worst = max(worst, compare_sequence(dec, m, i, ref, 0, ids if m["n_experts"] else None, tw,
                                                logits, out, pos + i, _pool_slot))
        nxt = int(out[C - 1])
        dec.close()
        pos += C
        flush(f"  chunk of {C} rows matches the oracle's {C} decode steps (worst rel err {worst:.2e})")
    # decode on over the prefilled pages
    dec = Decoder(m, W, kvpool, n_pages, [pos], [row], max_pages, pos + n_decode)
    tok = torch.tensor([nxt], dtype=torch.int32, device="cuda")
    ids = torch.full((L, 1, K), -1, dtype=torch.int32, device="cuda")
    tw = torch.zeros((L, 1, K), dtype=torch.float32, device="cuda")
    logits = torch.zeros((1, V), dtype=torch.float32, device="cuda")
    for s in range(n_decode):
        out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        dec.step(tok, out, ids if m["n_experts"] else None, tw if m["n_experts"] else None, logits)
        torch.cuda.synchronize()
        dec.check_status()
        ref, _, differ = O.decode_step_following(m, Wh, kv, [int(tok[0])],
                                                 [gpu_routing(ids, 0)] if m["n_experts"] else None, NEAR_TIE)
        assert not differ
        worst = max(worst, compare_sequence(dec, m, 0, ref, 0, ids if m["n_experts"] else None, tw, logits,
                                            out, pos + s, _pool_slot))
        tok = out
    flush(f"  {n_decode} decode steps over the prefilled pages match (worst rel err {worst:.2e})")
    dec.close()
    mk.mk_pool_free(pool)


def test_small_moe_chunk_across_a_page():
    run_prefill("small_moe", 100, [20], 4)


def test_small_moe_full_chunk_from_empty():
    run_prefill("small_moe", 0, [32], 2)


def test_tiny_dense_two_chunks():
    run_prefill("tiny_dense", 37, [13, 32], 3)


def test_moe48_chunk_after_8k():
    run_prefill("moe48_b1_8k", 8192, [16], 2, weights_from_device=True)
