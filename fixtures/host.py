"""ctypes wrapper of the host generator (fixtures/fx_host.c)."""
import ctypes
import os

import numpy as np
import torch

_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB = None

FX_EMBED, FX_ATTN_NORM, FX_WQKV, FX_WO, FX_FFN_NORM = 1, 2, 3, 4, 5
FX_ROUTER, FX_GATE, FX_UP, FX_DOWN, FX_FINAL_NORM = 6, 7, 8, 9, 10
FX_LM_HEAD, FX_KCACHE, FX_VCACHE, FX_TOKEN, FX_CTX, FX_PERM = 11, 12, 13, 14, 15, 16


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_DIR, "libfx.so")
        if not os.path.exists(path):
            raise RuntimeError("fixtures/libfx.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        u64, u32, f32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
        L.fx_mix64.restype = u64; L.fx_mix64.argtypes = [u64]
        L.fx_stream.restype = u64; L.fx_stream.argtypes = [u64, u64]
        L.fx_tag.restype = u64; L.fx_tag.argtypes = [u64, u64, u64, u64]
        L.fx_key.restype = u64; L.fx_key.argtypes = [u64, u64]
        L.fx_normal_f32.restype = f32; L.fx_normal_f32.argtypes = [u64, u64, f32]
        L.fx_bf16_rne.restype = ctypes.c_uint16; L.fx_bf16_rne.argtypes = [f32]
        L.fx_uniform.restype = u32; L.fx_uniform.argtypes = [u64, u64, u32, u32]
        L.fx_fill_normal_bf16.restype = None
        L.fx_fill_normal_bf16.argtypes = [ctypes.c_void_p, u64, u64, u64, f32]
        L.fx_permutation.restype = None
        L.fx_permutation.argtypes = [ctypes.c_void_p, ctypes.c_int32, u64]
        L.fx_uniform_fill.restype = None
        L.fx_uniform_fill.argtypes = [ctypes.c_void_p, u64, u64, u64, u32, u32]
        L.fx_threads.restype = ctypes.c_int
        _LIB = L
    return _LIB


def key(seed, kind, layer=0, a=0, b=0):
    L = lib()
    return L.fx_key(seed, L.fx_tag(kind, layer, a, b))


def normal_bf16(seed, kind, layer, a, b, i0, n, sigma):
    """bf16 bit patterns (torch.bfloat16 CPU tensor, 1-D) of elements [i0, i0+n)."""
    out = np.empty(n, dtype=np.uint16)
    if n:
        lib().fx_fill_normal_bf16(out.ctypes.data, key(seed, kind, layer, a, b), i0, n, sigma)
    return torch.from_numpy(out).view(torch.bfloat16)


def uniform(seed, kind, n, lo, hi):
    out = np.empty(n, dtype=np.uint32)
    if n:
        lib().fx_uniform_fill(out.ctypes.data, key(seed, kind), 0, n, lo, hi)
    return out


def permutation(seed, n):
    out = np.empty(n, dtype=np.int32)
    if n:
        lib().fx_permutation(out.ctypes.data, n, key(seed, FX_PERM))
    return out
