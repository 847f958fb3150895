"""Device-memory plumbing around the C ABI: a planned batch ready to step.

PyTorch provides device memory and the stream; every computation of the
decode step runs in libmk.so's kernels, and the plan, page bookkeeping and
rotary tables come from the library's host code. Nothing here computes any
part of the step.
"""
import ctypes

import numpy as np
import torch

from . import (
    MK_BUF_O, MK_BUF_Q, MK_BUF_RLOG, MK_BUF_XATTN, MK_BUF_XFFN,
    MK_PLAN_ATTN_QUEUE, MK_PLAN_NO_ROUTER_FOLD, MK_PLAN_CHANGED_COUNTERS, MK_PLAN_CHANGED_IMAGE, MK_PLAN_CHANGED_WORKSPACE,
    MkError, MK_OK, mk_decode_step, mk_decode_step_static, mk_io, mk_kv, mk_kv_pool_elems, mk_plan,
    mk_plan_buffer, mk_plan_counter_bytes, mk_plan_device_bytes, mk_plan_free, mk_plan_n_tasks,
    mk_plan_update, mk_plan_upload, mk_plan_workspace_bytes, mk_rope_table, mk_step_buffers, mk_stream_copy, mk_router_fold, mk_expert_tile,
    mk_sampling, mk_step_status, mk_weights, model_desc,
)

TRACE_WORDS = 16    # u64 per task in the optional trace buffer
CTR_LINES = 8       # sub-counters (64-byte lines) per completion counter


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def rope_tables(model, n_pos, device):
    """Rotary cos/sin tables [n_pos][head_dim/2] from the library, moved to the device."""
    h = model["head_dim"] // 2
    c = np.empty(n_pos * h, dtype=np.float32)
    s = np.empty(n_pos * h, dtype=np.float32)
    mk_rope_table(model["rope_theta"], model["head_dim"], n_pos, c.ctypes.data, s.ctypes.data)
    return (torch.from_numpy(c).view(n_pos, h).to(device), torch.from_numpy(s).view(n_pos, h).to(device))


def alloc_kv_pool(model, n_pages, device, zero=True):
    desc = model_desc(model)
    n = mk_kv_pool_elems(desc, n_pages)
    mk = torch.zeros if zero else torch.empty
    return mk(n, dtype=torch.bfloat16, device=device)


def copy_kv_page(model, pool, src, dst):
    """Copy KV page src to page dst of a device pool (every layer of the page;
    a page is contiguous in the pool layout), in stream order: the private
    copy of the page a shared prefix ends inside."""
    n = mk_kv_pool_elems(model_desc(model), 1) * pool.element_size()
    base = pool.data_ptr()
    mk_stream_copy(base + dst * n, base + src * n, n, torch.cuda.current_stream(pool.device).cuda_stream)


class Decoder:
    """A plan for one batch shape plus every device buffer a step needs.

    model: dict with the mk_model_desc field names. weights: dict of device
    bf16 tensors (fixtures.device.weights layout). pool: bf16 KV pool tensor.
    seq_lens: host ints (tokens cached per sequence). page_table: host
    [batch][max_pages] ints. bound: the plan stays valid while every
    sequence's length + 1 <= bound; ctx_bounds: per-sequence bounds (each
    <= bound), or None.
    """

    def __init__(self, model, weights, pool, n_pages, seq_lens, page_table, max_pages, bound,
                 n_cu=0, attn_split_pages=0, device="cuda", trace=False, plan_flags=0,
                 ctx_bounds=None, expert_tiles=True):
        self.m = dict(model)
        self.device = torch.device(device)
        self.B = len(seq_lens)
        self.desc = model_desc(self.m)
        self.plan_flags = plan_flags
        flat = [int(v) for row in page_table for v in row]
        self.plan = mk_plan(self.desc, seq_lens, flat, max_pages, bound, n_cu, attn_split_pages, plan_flags,
                            ctx_bounds)
        self.bound = bound
        dev = self.device
        self.plan_buf = torch.empty(mk_plan_device_bytes(self.plan), dtype=torch.uint8, device=dev)
        # tagged activation words: zero-filled once, then every step uses a larger epoch
        self.ws = torch.zeros(mk_plan_workspace_bytes(self.plan), dtype=torch.uint8, device=dev)
        self.ctr = torch.zeros(mk_plan_counter_bytes(self.plan) // 4, dtype=torch.int32, device=dev)
        self.status = torch.zeros(4, dtype=torch.int32, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        mk_plan_upload(self.plan, self.plan_buf.data_ptr(), self.plan_buf.numel(), stream)
        self.page_table = torch.tensor(flat, dtype=torch.int32, device=dev).view(self.B, max_pages)
        self.seq_lens = torch.tensor([int(v) for v in seq_lens], dtype=torch.int32, device=dev)
        self.pool = pool
        self.n_pages = n_pages
        self.W = weights
        self.epoch = 0
        # batch-1 MoE plans read the folded router W_r diag(g) W_o: made once
        # per weight set and kept in the weights dict
        self.router_folded = (self.B == 1 and self.m["n_experts"] > 0
                              and not (plan_flags & MK_PLAN_NO_ROUTER_FOLD))
        if self.router_folded and weights.get("router_fold") is None:
            m = self.m
            fold = torch.empty((m["n_layers"], m["n_experts"], m["hidden"] + m["n_q_heads"] * m["head_dim"]),
                               dtype=torch.float32, device=dev)
            w0 = mk_weights(*[_ptr(weights.get(k)) for k, _ in mk_weights._fields_])
            mk_router_fold(self.desc, w0, fold.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
            weights["router_fold"] = fold
        # batch plans' expert GEMMs read the expert weights in MFMA tile order
        # (mk_expert_tile): made once per weight set and kept in the weights dict
        self.expert_tiled = self.B > 1 and expert_tiles
        if self.expert_tiled and weights.get("expert_tiles") is None:
            m = self.m
            moe = m["n_experts"] > 0
            E = m["n_experts"] if moe else 1
            F = m["expert_ffn"] if moe else m["ffn_dim"]
            tiles = torch.empty(m["n_layers"] * E * 3 * F * m["hidden"], dtype=torch.bfloat16, device=dev)
            w0 = mk_weights(*[_ptr(weights.get(k)) for k, _ in mk_weights._fields_])
            mk_expert_tile(self.desc, w0, tiles.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
            weights["expert_tiles"] = tiles
        self._w = mk_weights(*[_ptr(weights.get(k)) if (k != "expert_tiles" or self.expert_tiled) else None
                               for k, _ in mk_weights._fields_])
        self._set_rope(bound)
        self.trace = None
        if trace:
            n = mk_plan_n_tasks(self.plan) * TRACE_WORDS
            self.trace = torch.zeros(n, dtype=torch.int64, device=dev)
        self._set_bufs()

    def _set_rope(self, n_pos):
        self.rope_cos, self.rope_sin = rope_tables(self.m, n_pos, self.device)
        self._kv = mk_kv(self.pool.data_ptr(), self.n_pages, self.page_table.data_ptr(),
                         self.seq_lens.data_ptr(), self.rope_cos.data_ptr(),
                         self.rope_sin.data_ptr(), n_pos)

    def _set_bufs(self):
        self._bufs = mk_step_buffers(self.plan_buf.data_ptr(), self.plan_buf.numel(),
                                     self.ws.data_ptr(), self.ws.numel(), self.ctr.data_ptr(),
                                     self.ctr.numel() * 4, self.status.data_ptr(),
                                     _ptr(self.trace),
                                     0 if self.trace is None else self.trace.numel() * 8)

    def update(self, seq_lens, page_table, bound, ctx_bounds=None):
        """Refresh the plan for new lengths / page table / bounds of the same
        batch (mk_plan_update) and apply what changed, in stream order after
        the steps already enqueued: the device image, a fresh workspace,
        counters and epochs where the planner asks for them, the device page
        table and lengths, and larger rope tables if the bound outgrew them.
        Returns the MK_PLAN_CHANGED_* bits."""
        flat = [int(v) for row in page_table for v in row]
        ch = mk_plan_update(self.plan, seq_lens, flat, bound, ctx_bounds)
        dev = self.device
        stream = torch.cuda.current_stream(dev).cuda_stream
        if ch & MK_PLAN_CHANGED_IMAGE:
            n = mk_plan_device_bytes(self.plan)
            if n > self.plan_buf.numel():
                self.plan_buf = torch.empty(n, dtype=torch.uint8, device=dev)
            mk_plan_upload(self.plan, self.plan_buf.data_ptr(), self.plan_buf.numel(), stream)
        if ch & (MK_PLAN_CHANGED_WORKSPACE | MK_PLAN_CHANGED_COUNTERS):
            nw, nc = mk_plan_workspace_bytes(self.plan), mk_plan_counter_bytes(self.plan) // 4
            if nw != self.ws.numel():
                self.ws = torch.zeros(nw, dtype=torch.uint8, device=dev)
            else:
                self.ws.zero_()
            if nc != self.ctr.numel():
                self.ctr = torch.zeros(nc, dtype=torch.int32, device=dev)
            else:
                self.ctr.zero_()
            self.epoch = 0
            if self.trace is not None:
                n = mk_plan_n_tasks(self.plan) * TRACE_WORDS
                self.trace = torch.zeros(n, dtype=torch.int64, device=dev)
        self.page_table.copy_(torch.tensor(flat, dtype=torch.int32).view_as(self.page_table))
        self.seq_lens.copy_(torch.tensor([int(v) for v in seq_lens], dtype=torch.int32))
        if bound > self._kv.n_rope_pos:
            self._set_rope(bound)
        self.bound = bound
        self._set_bufs()
        return ch

    def close(self):
        if self.plan:
            mk_plan_free(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, tokens_in, tokens_out, topk_ids=None, topk_w=None, logits=None, timeout_ms=0,
             sampling=None):
        """Enqueue one decode step on the current stream (asynchronous).
        sampling: None (greedy), or a dict of device [batch] tensors
        temperature (f32), top_k (i32), top_p (f32), min_p (f32), uniform (f32)."""
        self.epoch += 1
        io = mk_io(_ptr(tokens_in), _ptr(tokens_out), _ptr(topk_ids), _ptr(topk_w), _ptr(logits))
        if sampling is not None:
            self._smp = mk_sampling(*[_ptr(sampling[k]) for k, _ in mk_sampling._fields_])
            io.sampling = ctypes.pointer(self._smp)
        mk_decode_step(self.plan, self._w, self._kv, io, self._bufs, self.epoch, timeout_ms,
                       torch.cuda.current_stream(self.device).cuda_stream)

    def step_static(self, tokens_in, tokens_out, topk_ids=None, topk_w=None, logits=None, timeout_ms=0):
        """Enqueue one decode step through the allocation-free entry point:
        the workspace and counters live in the library's static scratch
        (this decoder's own workspace, counters and epochs are not used)."""
        io = mk_io(_ptr(tokens_in), _ptr(tokens_out), _ptr(topk_ids), _ptr(topk_w), _ptr(logits))
        mk_decode_step_static(self.plan, self._w, self._kv, io, self.plan_buf.data_ptr(), self.plan_buf.numel(),
                              self.status.data_ptr(), timeout_ms,
                              torch.cuda.current_stream(self.device).cuda_stream)

    def recover(self, seq_lens):
        """Make the decoder usable after a failed step (status words set):
        zero the status and counters, put back the sequence lengths of
        before the step and, with the attention queue, start again from a
        zero-filled workspace and epoch 1. The next step uses a new epoch."""
        self.status.zero_()
        self.ctr.zero_()
        self.seq_lens.copy_(torch.tensor([int(v) for v in seq_lens], dtype=torch.int32))
        if self.plan_flags & MK_PLAN_ATTN_QUEUE:
            self.ws.zero_()
            self.epoch = 0

    def check_status(self):
        """Synchronise and raise MkError if the device recorded a failure."""
        h = self.status.cpu().tolist()
        st, msg = mk_step_status([v & 0xFFFFFFFF for v in h])
        if st != MK_OK:
            raise MkError(st, msg)

    def counters(self):
        """Completion counts per counter (sum of its lines modulo 2^32), as a host int64 tensor."""
        c = self.ctr.view(-1, CTR_LINES, 16)[:, :, 0].to(torch.int64) & 0xFFFFFFFF
        return c.sum(dim=1).cpu() % (1 << 32)

    def buffer(self, which, layer=0):
        """Workspace sub-buffer (MK_BUF_*) of one layer: its tagged u64 words (device view)."""
        off, nb = mk_plan_buffer(self.plan, which, layer)
        return self.ws[off:off + nb].view(torch.int64)

    def values(self, which, layer=0):
        """(values fp32, tags int64) of a tagged sub-buffer, on the host."""
        w = self.buffer(which, layer).cpu()
        vals = (w & 0xFFFFFFFF).to(torch.int32).view(torch.float32)
        tags = (w >> 32) & 0xFFFFFFFF
        return vals, tags

    def _current(self, which, layer, shape):
        v, t = self.values(which, layer)
        if not bool((t == self.epoch).all()):
            raise RuntimeError(f"buffer {which} layer {layer} holds words of another step")
        return v.view(*shape)

    def hidden_after_attn(self, layer):
        return self._current(MK_BUF_XATTN, layer, (self.B, self.m["hidden"]))

    def hidden_after_ffn(self, layer):
        return self._current(MK_BUF_XFFN, layer, (self.B, self.m["hidden"]))

    def router_logits(self, layer):
        """Router logits [B][E]. A folded router stores them before the
        RMSNorm's 1/rms of the hidden state after attention, applied here."""
        r = self._current(MK_BUF_RLOG, layer, (self.B, self.m["n_experts"]))
        if self.router_folded:
            x = self.hidden_after_attn(layer).double()
            r = (r.double() / torch.sqrt((x * x).mean(dim=1, keepdim=True) + self.m["rms_eps"])).float()
        return r

    def queries(self, layer):
        return self._current(MK_BUF_Q, layer, (self.B, self.m["n_q_heads"], self.m["head_dim"]))

    def attn_out(self, layer):
        return self._current(MK_BUF_O, layer, (self.B, self.m["n_q_heads"], self.m["head_dim"]))
