"""Host-side (CPU) synthetic weights and contiguous prior KV, for the oracle.

Tensors are generated on first use and cached; logical layouts are plain
row-major [out][in] matrices and contiguous K, V of shape [tokens][head_dim].
"""
import torch

from . import host
from .workloads import SIGMA_W, SIGMA_KV


class HostWeights:
    """Lazily generated bf16 weights (torch CPU tensors) of one model."""

    def __init__(self, model, seed=0, cache=True):
        self.m = dict(model)
        self.seed = seed
        self.cache = cache
        self._c = {}

    def _gen(self, kind, layer, a, rows, cols):
        k = (kind, layer, a)
        if k in self._c:
            return self._c[k]
        t = host.normal_bf16(self.seed, kind, layer, a, 0, 0, rows * cols, SIGMA_W).view(rows, cols)
        if self.cache:
            self._c[k] = t
        return t

    def norm(self, n):
        return torch.ones(n, dtype=torch.bfloat16)

    # --- per-tensor accessors (logical layouts) ---
    def embed_row(self, tok):
        m = self.m
        return host.normal_bf16(self.seed, host.FX_EMBED, 0, 0, 0, tok * m["hidden"], m["hidden"], SIGMA_W)

    def attn_norm(self, l):
        return self.norm(self.m["hidden"])

    def ffn_norm(self, l):
        return self.norm(self.m["hidden"])

    def final_norm(self):
        return self.norm(self.m["hidden"])

    def wqkv(self, l):
        m = self.m
        rows = (m["n_q_heads"] + 2 * m["n_kv_heads"]) * m["head_dim"]
        return self._gen(host.FX_WQKV, l, 0, rows, m["hidden"])

    def wo(self, l):
        m = self.m
        return self._gen(host.FX_WO, l, 0, m["hidden"], m["n_q_heads"] * m["head_dim"])

    def router(self, l):
        m = self.m
        return self._gen(host.FX_ROUTER, l, 0, m["n_experts"], m["hidden"])

    def gate(self, l, e=0):
        m = self.m
        f = m["expert_ffn"] if m["n_experts"] else m["ffn_dim"]
        return self._gen(host.FX_GATE, l, e, f, m["hidden"])

    def up(self, l, e=0):
        m = self.m
        f = m["expert_ffn"] if m["n_experts"] else m["ffn_dim"]
        return self._gen(host.FX_UP, l, e, f, m["hidden"])

    def down(self, l, e=0):
        m = self.m
        f = m["expert_ffn"] if m["n_experts"] else m["ffn_dim"]
        return self._gen(host.FX_DOWN, l, e, m["hidden"], f)

    def lm_head(self):
        m = self.m
        return self._gen(host.FX_LM_HEAD, 0, 0, m["vocab"], m["hidden"])


class HostKV:
    """Prior KV of sequence b, layer l, kv head g as contiguous bf16 [ctx][d]."""

    def __init__(self, model, seed=0):
        self.m = dict(model)
        self.seed = seed

    def k(self, l, b, g, ctx):
        d = self.m["head_dim"]
        return host.normal_bf16(self.seed, host.FX_KCACHE, l, b, g, 0, ctx * d, SIGMA_KV).view(ctx, d)

    def v(self, l, b, g, ctx):
        d = self.m["head_dim"]
        return host.normal_bf16(self.seed, host.FX_VCACHE, l, b, g, 0, ctx * d, SIGMA_KV).view(ctx, d)


class DeviceCopyWeights(HostWeights):
    """The same weights, copied to the host from the device tensors that
    fixtures.device.weights filled (the device implementation of the same
    generator, pinned bit for bit to the host one by a GPU test). Reading
    back is much faster than drawing tens of GB again on the host; the
    values are the generator's, not any result of the decode step."""

    def __init__(self, model, dev_weights, seed=0, cache=True):
        super().__init__(model, seed, cache)
        self.D = dev_weights

    def _get(self, key, fn):
        if key in self._c:
            return self._c[key]
        t = fn().cpu()
        if self.cache:
            self._c[key] = t
        return t

    def embed_row(self, tok):
        return self.D["embed"][tok].cpu()

    def wqkv(self, l):
        return self._get(("wqkv", l), lambda: self.D["w_qkv"][l])

    def wo(self, l):
        return self._get(("wo", l), lambda: self.D["w_o"][l])

    def router(self, l):
        return self._get(("router", l), lambda: self.D["router"][l])

    def gate(self, l, e=0):
        return self._get(("gate", l, e), lambda: self.D["gate"][l, e])

    def up(self, l, e=0):
        return self._get(("up", l, e), lambda: self.D["up"][l, e])

    def down(self, l, e=0):
        return self._get(("down", l, e), lambda: self.D["down"][l, e])

    def lm_head(self):
        return self._get(("lm",), lambda: self.D["lm_head"])
