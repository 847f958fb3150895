"""Python binding of libmk.so (include/mk.h): argument marshalling only.

Every function here has the name of the C entry point it calls and raises
MkError (with mk_last_error()) when the call fails. All arithmetic of the
decode step runs in the HIP kernels of libmk.so; importing this package
fails loudly if the library has not been built.
"""
import ctypes
import os

_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_DIR, "libmk.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError("libmk.so is not built: run `python __graft_entry__.py` (build()) first")
_lib = ctypes.CDLL(_LIB_PATH)

MK_OK, MK_EINVAL, MK_ENOMEM, MK_EBOUNDS, MK_EDEVICE, MK_ETIMEOUT, MK_ESTATE, MK_EUNSUPPORTED = (
    0, -1, -2, -3, -4, -5, -6, -7)
STATUS_NAMES = {0: "MK_OK", -1: "MK_EINVAL", -2: "MK_ENOMEM", -3: "MK_EBOUNDS", -4: "MK_EDEVICE",
                -5: "MK_ETIMEOUT", -6: "MK_ESTATE", -7: "MK_EUNSUPPORTED"}
(MK_BUF_XATTN, MK_BUF_XFFN, MK_BUF_Q, MK_BUF_PART, MK_BUF_O, MK_BUF_RLOG, MK_BUF_ACT,
 MK_BUF_LMPART, MK_BUF_KVN, MK_BUF_ROUTE, MK_BUF_Y, MK_BUF_OPART, MK_BUF_QPART, MK_BUF_LOGIT) = range(14)

_i32, _i64, _u32, _u64, _f32, _sz, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                         ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t,
                                         ctypes.c_void_p)


class MkError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class mk_model_desc(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                    "ffn_dim", "n_experts", "top_k", "expert_ffn", "norm_topk",
                                    "vocab", "page_tokens")] + [("rms_eps", _f32), ("rope_theta", _f32)]


class mk_batch_desc(ctypes.Structure):
    _fields_ = [("batch", _i32), ("max_pages", _i32), ("seq_lens", ctypes.POINTER(_i32)),
                ("page_table", ctypes.POINTER(_i32)), ("max_ctx_bound", _i32),
                ("ctx_bounds", ctypes.POINTER(_i32))]


class mk_plan_opts(ctypes.Structure):
    _fields_ = [("n_cu", _i32), ("attn_split_pages", _i32), ("flags", _i32)]


class mk_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("embed", "attn_norm", "w_qkv", "w_o", "ffn_norm", "router",
                                   "gate", "up", "down", "final_norm", "lm_head", "router_fold",
                                   "expert_tiles")]


class mk_kv(ctypes.Structure):
    _fields_ = [("pool", _vp), ("n_pages", _i64), ("page_table", _vp), ("seq_lens", _vp),
                ("rope_cos", _vp), ("rope_sin", _vp), ("n_rope_pos", _i32)]


class mk_sampling(ctypes.Structure):
    _fields_ = [("temperature", _vp), ("top_k", _vp), ("top_p", _vp), ("min_p", _vp), ("uniform", _vp)]


class mk_io(ctypes.Structure):
    _fields_ = [("tokens_in", _vp), ("tokens_out", _vp), ("topk_ids", _vp), ("topk_w", _vp),
                ("logits", _vp), ("sampling", ctypes.POINTER(mk_sampling))]


MK_SAMPLE_TOP_K_MAX = 64


class mk_step_buffers(ctypes.Structure):
    _fields_ = [("plan", _vp), ("plan_bytes", _sz), ("workspace", _vp), ("workspace_bytes", _sz),
                ("counters", _vp), ("counter_bytes", _sz), ("status", _vp),
                ("trace", _vp), ("trace_bytes", _sz)]


_P = ctypes.POINTER
_SIGS = {
    "mk_abi_version": (_i32, []),
    "mk_last_error": (ctypes.c_char_p, []),
    "mk_device_cu_count": (_i32, [_P(_i32)]),
    "mk_stream_copy": (_i32, [_vp, _vp, _sz, _vp]),
    "mk_router_fold": (_i32, [_vp, _vp, _vp, _vp]),
    "mk_expert_tile": (_i32, [_vp, _vp, _vp, _vp]),
    "mk_rope_table": (_i32, [_f32, _i32, _i32, _vp, _vp]),
    "mk_kv_pool_elems": (_i64, [_P(mk_model_desc), _i64]),
    "mk_step_bytes": (_i32, [_P(mk_model_desc), _i32, _P(_i32), _P(_i32), _P(ctypes.c_double),
                             _P(ctypes.c_double), _P(ctypes.c_double)]),
    "mk_plan": (_i32, [_P(mk_model_desc), _P(mk_batch_desc), _P(mk_plan_opts), _P(_vp)]),
    "mk_plan_update": (_i32, [_vp, _P(_i32), _P(_i32), _i32, _P(_i32), _P(_i32)]),
    "mk_plan_validate": (_i32, [_vp]),
    "mk_plan_simulate": (_i32, [_vp, _u64, _i32]),
    "mk_plan_device_bytes": (_sz, [_vp]),
    "mk_plan_workspace_bytes": (_sz, [_vp]),
    "mk_plan_counter_bytes": (_sz, [_vp]),
    "mk_plan_n_tasks": (_i32, [_vp]),
    "mk_plan_n_counters": (_i32, [_vp]),
    "mk_plan_n_cu": (_i32, [_vp]),
    "mk_plan_export": (_i32, [_vp, _vp, _sz]),
    "mk_plan_upload": (_i32, [_vp, _vp, _sz, _vp]),
    "mk_plan_buffer": (_i32, [_vp, _i32, _i32, _P(_sz), _P(_sz)]),
    "mk_plan_counter_targets": (_i32, [_vp, _vp, _i32]),
    "mk_plan_counter_name": (ctypes.c_char_p, [_vp, _i32]),
    "mk_plan_free": (None, [_vp]),
    "mk_decode_step": (_i32, [_vp, _P(mk_weights), _P(mk_kv), _P(mk_io), _P(mk_step_buffers),
                              _u32, _u32, _vp]),
    "mk_decode_step_static": (_i32, [_vp, _P(mk_weights), _P(mk_kv), _P(mk_io), _vp, _sz, _vp, _u32, _vp]),
    "mk_step_status": (_i32, [_vp]),
    "mk_pool_create": (_i32, [_i32, _i32, _i32, _vp, _P(_vp)]),
    "mk_pool_lease": (_i32, [_vp, _i64, _i32, _P(_i32)]),
    "mk_pool_lease_prefix": (_i32, [_vp, _i64, _vp, _i32, _i32, _P(_i32), _P(_i32), _P(_i32), _P(_i32)]),
    "mk_pool_finish": (_i32, [_vp, _i64, _vp, _i32]),
    "mk_pool_cached_pages": (_i32, [_vp]),
    "mk_pool_extend": (_i32, [_vp, _i64, _i32]),
    "mk_pool_release": (_i32, [_vp, _i64]),
    "mk_pool_page_table": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "mk_pool_free_pages": (_i32, [_vp]),
    "mk_pool_seq_pages": (_i32, [_vp, _i64]),
    "mk_pool_free": (None, [_vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def mk_last_error():
    return _lib.mk_last_error().decode()


def _check(st):
    if st != MK_OK:
        raise MkError(st, mk_last_error())
    return st


def mk_abi_version():
    return _lib.mk_abi_version()


def mk_device_cu_count():
    n = _i32()
    _check(_lib.mk_device_cu_count(ctypes.byref(n)))
    return n.value


def mk_router_fold(desc, weights, out_ptr, stream_ptr):
    """out = W_r diag(ffn_norm) W_o per layer (fp32 [L][E][Hq d], device)."""
    _check(_lib.mk_router_fold(ctypes.byref(desc), ctypes.byref(weights), out_ptr, stream_ptr))


def mk_expert_tile(desc, weights, out_ptr, stream_ptr):
    """Fill out_ptr (device) with the expert weights in MFMA tile order (mk.h)."""
    _check(_lib.mk_expert_tile(ctypes.byref(desc), ctypes.byref(weights), out_ptr, stream_ptr))


def mk_stream_copy(dst_ptr, src_ptr, nbytes, stream_ptr):
    _check(_lib.mk_stream_copy(dst_ptr, src_ptr, nbytes, stream_ptr))


def model_desc(m):
    """mk_model_desc from a dict with the mk_model_desc field names."""
    return mk_model_desc(**{k: m[k] for k, _ in mk_model_desc._fields_})


def mk_rope_table(theta, head_dim, n_pos, cos_ptr, sin_ptr):
    _check(_lib.mk_rope_table(theta, head_dim, n_pos, cos_ptr, sin_ptr))


def mk_kv_pool_elems(desc, n_pages):
    return _lib.mk_kv_pool_elems(ctypes.byref(desc), n_pages)


def mk_step_bytes(desc, seq_lens, distinct=None):
    B = len(seq_lens)
    sl = (_i32 * B)(*seq_lens)
    de = (_i32 * len(distinct))(*distinct) if distinct is not None else None
    w, r, wr = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(_lib.mk_step_bytes(ctypes.byref(desc), B, sl, de, ctypes.byref(w), ctypes.byref(r),
                              ctypes.byref(wr)))
    return w.value, r.value, wr.value


_plan_shape = {}   # plan handle -> (batch, page-table width), for mk_plan_update's argument check

MK_PLAN_ATTN_QUEUE = 1
MK_PLAN_NO_ATTN_QUEUE = 2
MK_PLAN_PREFILL = 4
MK_PLAN_NO_ROUTER_FOLD = 8
MK_PLAN_NO_EXPERT_SHARE = 16


def mk_plan(desc, seq_lens, page_table, max_pages, bound, n_cu=0, attn_split_pages=0, flags=0,
            ctx_bounds=None):
    """Build a plan. page_table: flat host list/array of batch*max_pages int32;
    ctx_bounds: per-sequence context bounds, or None (every sequence: bound)."""
    B = len(seq_lens)
    sl = (_i32 * B)(*[int(v) for v in seq_lens])
    pt = (_i32 * (B * max_pages))(*[int(v) for v in page_table])
    cb = (_i32 * B)(*[int(v) for v in ctx_bounds]) if ctx_bounds is not None else None
    bd = mk_batch_desc(B, max_pages, sl, pt, bound, cb)
    op = mk_plan_opts(n_cu, attn_split_pages, flags)
    out = _vp()
    _check(_lib.mk_plan(ctypes.byref(desc), ctypes.byref(bd), ctypes.byref(op), ctypes.byref(out)))
    _plan_shape[out.value] = (B, max_pages)
    return out.value


MK_PLAN_CHANGED_IMAGE, MK_PLAN_CHANGED_WORKSPACE, MK_PLAN_CHANGED_COUNTERS = 1, 2, 4


def mk_plan_update(p, seq_lens, page_table, bound, ctx_bounds=None):
    """Refresh plan p in place; returns the MK_PLAN_CHANGED_* bits."""
    B = len(seq_lens)
    if (B, len(page_table) // max(B, 1)) != _plan_shape.get(p) or len(page_table) % max(B, 1) \
            or (ctx_bounds is not None and len(ctx_bounds) != B):
        raise ValueError(f"mk_plan_update: batch {B} / page table of {len(page_table)} entries do not match "
                         f"the plan's (batch, pages per row) {_plan_shape.get(p)}")
    sl = (_i32 * B)(*[int(v) for v in seq_lens])
    pt = (_i32 * len(page_table))(*[int(v) for v in page_table])
    cb = (_i32 * B)(*[int(v) for v in ctx_bounds]) if ctx_bounds is not None else None
    ch = _i32()
    _check(_lib.mk_plan_update(p, sl, pt, bound, cb, ctypes.byref(ch)))
    return ch.value


def mk_plan_validate(p):
    return _check(_lib.mk_plan_validate(p))


def mk_plan_simulate(p, seed, n_runs):
    return _check(_lib.mk_plan_simulate(p, seed, n_runs))


def mk_plan_device_bytes(p):
    return _lib.mk_plan_device_bytes(p)


def mk_plan_workspace_bytes(p):
    return _lib.mk_plan_workspace_bytes(p)


def mk_plan_counter_bytes(p):
    return _lib.mk_plan_counter_bytes(p)


def mk_plan_n_tasks(p):
    return _lib.mk_plan_n_tasks(p)


def mk_plan_n_counters(p):
    return _lib.mk_plan_n_counters(p)


def mk_plan_n_cu(p):
    return _lib.mk_plan_n_cu(p)


def mk_plan_export(p):
    n = _lib.mk_plan_device_bytes(p)
    buf = (ctypes.c_uint8 * n)()
    _check(_lib.mk_plan_export(p, buf, n))
    return bytes(buf)


def mk_plan_upload(p, d_ptr, nbytes, stream):
    _check(_lib.mk_plan_upload(p, d_ptr, nbytes, stream))


def mk_plan_buffer(p, which, layer):
    off, nb = _sz(), _sz()
    _check(_lib.mk_plan_buffer(p, which, layer, ctypes.byref(off), ctypes.byref(nb)))
    return off.value, nb.value


def mk_plan_counter_targets(p):
    n = _lib.mk_plan_n_counters(p)
    buf = (_u32 * n)()
    _check(_lib.mk_plan_counter_targets(p, buf, n))
    return list(buf)


def mk_plan_counter_name(p, i):
    r = _lib.mk_plan_counter_name(p, i)
    if r is None:
        raise MkError(MK_EINVAL, mk_last_error())
    return r.decode()


def mk_plan_counter_names(p):
    return [mk_plan_counter_name(p, i) for i in range(_lib.mk_plan_n_counters(p))]


def mk_plan_free(p):
    _plan_shape.pop(p, None)
    _lib.mk_plan_free(p)


def mk_decode_step(p, weights, kv, io, bufs, epoch, timeout_ms, stream):
    _check(_lib.mk_decode_step(p, ctypes.byref(weights), ctypes.byref(kv), ctypes.byref(io),
                               ctypes.byref(bufs), epoch, timeout_ms, stream))


MK_STATIC_SCRATCH_BYTES = 128 << 20


def mk_decode_step_static(p, weights, kv, io, d_plan, plan_bytes, d_status, timeout_ms, stream):
    _check(_lib.mk_decode_step_static(p, ctypes.byref(weights), ctypes.byref(kv), ctypes.byref(io), d_plan,
                                      plan_bytes, d_status, timeout_ms, stream))


def mk_step_status(h_status4):
    """Decode 4 status words (sequence of ints). Returns (status, message)."""
    arr = (_u32 * 4)(*[int(v) for v in h_status4])
    st = _lib.mk_step_status(arr)
    return st, (mk_last_error() if st != MK_OK else "")


def mk_pool_create(n_pages, page_tokens, n_slots, initial_order=None):
    out = _vp()
    order = (_i32 * n_pages)(*[int(v) for v in initial_order]) if initial_order is not None else None
    _check(_lib.mk_pool_create(n_pages, page_tokens, n_slots, order, ctypes.byref(out)))
    return out.value


def mk_pool_lease(pool, seq_id, tokens):
    slot = _i32()
    _check(_lib.mk_pool_lease(pool, seq_id, tokens, ctypes.byref(slot)))
    return slot.value


def mk_pool_lease_prefix(pool, seq_id, prompt, tokens):
    """Lease with prefix sharing: returns (slot, matched tokens, copy_src, copy_dst)."""
    n = len(prompt)
    pr = (_i32 * max(n, 1))(*[int(v) for v in prompt])
    slot, m, cs, cd = _i32(), _i32(), _i32(), _i32()
    _check(_lib.mk_pool_lease_prefix(pool, seq_id, pr, n, tokens, ctypes.byref(slot), ctypes.byref(m),
                                     ctypes.byref(cs), ctypes.byref(cd)))
    return slot.value, m.value, cs.value, cd.value


def mk_pool_finish(pool, seq_id, tokens):
    n = len(tokens)
    tk = (_i32 * max(n, 1))(*[int(v) for v in tokens])
    _check(_lib.mk_pool_finish(pool, seq_id, tk, n))


def mk_pool_cached_pages(pool):
    return _lib.mk_pool_cached_pages(pool)


def mk_pool_extend(pool, seq_id, tokens):
    _check(_lib.mk_pool_extend(pool, seq_id, tokens))


def mk_pool_release(pool, seq_id):
    _check(_lib.mk_pool_release(pool, seq_id))


def mk_pool_page_table(pool, seq_ids, max_pages):
    n = len(seq_ids)
    ids = (_i64 * n)(*seq_ids)
    out = (_i32 * (n * max_pages))()
    _check(_lib.mk_pool_page_table(pool, ids, n, max_pages, out))
    return [list(out[i * max_pages:(i + 1) * max_pages]) for i in range(n)]


def mk_pool_free_pages(pool):
    return _lib.mk_pool_free_pages(pool)


def mk_pool_seq_pages(pool, seq_id):
    return _lib.mk_pool_seq_pages(pool, seq_id)


def mk_pool_free(pool):
    _lib.mk_pool_free(pool)


def kernel_hash():
    """Hash of the device sources (csrc/*.hip, *.hpp): hardware-counter figures
    recorded for one kernel build are valid only while it matches."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]
