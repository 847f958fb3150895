"""Device-resident synthetic inputs (torch tensors on a GPU), filled in place
by libfx_gpu.so with the generator defined in fx.h.

Test and benchmark infrastructure: it allocates weights and the paged KV
pool in the layouts the decode library documents (include/mk.h) and fills
them with the same values the host generator gives the oracle. It holds no
arithmetic of the decode step.
"""
import ctypes
import os

import torch

from . import host
from .workloads import SIGMA_W, SIGMA_KV, NORM_GAIN_BITS

_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_DIR, "libfx_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError("fixtures/libfx_gpu.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        u64, u32, f32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p
        L.fx_gpu_fill_normal_bf16.restype = ctypes.c_int
        L.fx_gpu_fill_normal_bf16.argtypes = [vp, u64, u64, u64, f32, vp]
        L.fx_gpu_fill_stack_bf16.restype = ctypes.c_int
        L.fx_gpu_fill_stack_bf16.argtypes = [vp, u64, u32, u32, u32, u32, u64, f32, vp]
        L.fx_gpu_fill_const_bf16.restype = ctypes.c_int
        L.fx_gpu_fill_const_bf16.argtypes = [vp, u64, ctypes.c_uint16, vp]
        L.fx_gpu_fill_kv.restype = ctypes.c_int
        L.fx_gpu_fill_kv.argtypes = [vp, vp, u64, u32, u32, u32, u32, u32, u32, u32, u32, vp]
        _LIB = L
    return _LIB


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def fill_stack(t, seed, kind, n_layers, n_sub, per, sigma=SIGMA_W):
    """t: bf16 [n_layers][n_sub][per] with matrix (l, e) = normal(key(seed, tag(kind, l, e, 0)))."""
    assert t.dtype == torch.bfloat16 and t.is_contiguous() and t.numel() == n_layers * n_sub * per
    _ok(lib().fx_gpu_fill_stack_bf16(t.data_ptr(), seed, kind, 0, n_layers, n_sub, per, sigma,
                                     _stream()), "fx_gpu_fill_stack_bf16")


def fill_const(t, bits):
    assert t.dtype == torch.bfloat16 and t.is_contiguous()
    _ok(lib().fx_gpu_fill_const_bf16(t.data_ptr(), t.numel(), bits, _stream()), "fx_gpu_fill_const_bf16")


def weights(m, seed=0, device="cuda"):
    """All weights of model m as device bf16 tensors in the library's layouts.

    Values equal fixtures.HostWeights(m, seed) element for element.
    """
    L, H, Hq, Hkv, d = m["n_layers"], m["hidden"], m["n_q_heads"], m["n_kv_heads"], m["head_dim"]
    moe = m["n_experts"] > 0
    E = m["n_experts"] if moe else 1
    F = m["expert_ffn"] if moe else m["ffn_dim"]
    V = m["vocab"]
    bf = dict(dtype=torch.bfloat16, device=device)
    W = {
        "embed": torch.empty(V, H, **bf),
        "attn_norm": torch.empty(L, H, **bf),
        "w_qkv": torch.empty(L, (Hq + 2 * Hkv) * d, H, **bf),
        "w_o": torch.empty(L, H, Hq * d, **bf),
        "ffn_norm": torch.empty(L, H, **bf),
        "router": torch.empty(L, E, H, **bf) if moe else None,
        "gate": torch.empty(L, E, F, H, **bf),
        "up": torch.empty(L, E, F, H, **bf),
        "down": torch.empty(L, E, H, F, **bf),
        "final_norm": torch.empty(H, **bf),
        "lm_head": torch.empty(V, H, **bf),
    }
    fill_stack(W["embed"], seed, host.FX_EMBED, 1, 1, V * H)
    fill_stack(W["w_qkv"], seed, host.FX_WQKV, L, 1, (Hq + 2 * Hkv) * d * H)
    fill_stack(W["w_o"], seed, host.FX_WO, L, 1, H * Hq * d)
    if moe:
        fill_stack(W["router"], seed, host.FX_ROUTER, L, 1, E * H)
    fill_stack(W["gate"], seed, host.FX_GATE, L, E, F * H)
    fill_stack(W["up"], seed, host.FX_UP, L, E, F * H)
    fill_stack(W["down"], seed, host.FX_DOWN, L, E, H * F)
    fill_stack(W["lm_head"], seed, host.FX_LM_HEAD, 1, 1, V * H)
    for k in ("attn_norm", "ffn_norm", "final_norm"):
        fill_const(W[k], NORM_GAIN_BITS)
    return W


def fill_kv(pool, page_row_dev, m, seed, b, ctx, start=0):
    """Prior KV of sequence b (tokens start .. ctx-1) into its pages of the device pool.

    page_row_dev: int32 device tensor, the sequence's row of the page table.
    Values equal fixtures.HostKV(m, seed).k / .v element for element; slots
    of tokens below start (e.g. pages shared with a checkpoint) are not written.
    """
    assert pool.dtype == torch.bfloat16 and page_row_dev.dtype == torch.int32
    n_pg = page_row_dev.numel()
    pt = m["page_tokens"]
    need = (ctx + pt - 1) // pt
    if need > n_pg:
        raise ValueError("fill_kv: page row shorter than the context")
    rows = page_row_dev[start // pt:need].cpu()
    n_pages = pool.numel() // (m["n_layers"] * m["n_kv_heads"] * 2 * pt * m["head_dim"])
    if rows.numel() and (int(rows.min()) < 0 or int(rows.max()) >= n_pages):
        raise ValueError("fill_kv: page id outside the pool")
    _ok(lib().fx_gpu_fill_kv(pool.data_ptr(), page_row_dev.data_ptr(), seed, b, start, ctx, n_pg,
                             m["n_layers"], m["n_kv_heads"], m["head_dim"], pt, _stream()),
        "fx_gpu_fill_kv")
