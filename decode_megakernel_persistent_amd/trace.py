"""Decode the optional per-task trace of a decode step.

The trace buffer (mk_step_buffers.trace) holds 16 u64 words per task, in
plan-image order: task start, routing-wait begin/end, data-wait begin/end
(0 where the task has no such wait), body end, task end (ticks of the
100 MHz constant clock), cu << 32 | op << 16 | layer, then 8 marks set by
the task body at points of its own (0 = unset). This module turns
it into per-operation time splits and a per-stage timeline.
"""
import numpy as np

OPS = {1: "qkv", 2: "attn", 3: "comb", 4: "o", 5: "router", 6: "expert", 8: "lm",
       9: "final", 10: "bqkv", 11: "bo", 13: "topk", 14: "bexp", 15: "bcomb", 16: "blm",
       17: "bfinal"}
TICK_US = 0.01  # 100 MHz


def decode(raw):
    """raw: int64 tensor/array of n_tasks * 8 words -> dict of numpy columns (us, relative)."""
    a = np.asarray(raw.cpu() if hasattr(raw, "cpu") else raw).view(np.uint64).reshape(-1, 16)
    t0 = a[:, 0].astype(np.float64)
    base = t0[t0 > 0].min()
    rel = lambda c: np.where(a[:, c] > 0, (a[:, c].astype(np.float64) - base) * TICK_US, np.nan)
    meta = a[:, 7]
    return {
        "start": rel(0), "wa0": rel(1), "wa1": rel(2), "wb0": rel(3), "wb1": rel(4),
        "body": rel(5), "end": rel(6),
        "cu": (meta >> np.uint64(32)).astype(np.int64),
        "op": ((meta >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.int64),
        "layer": (meta & np.uint64(0xFFFF)).astype(np.int64),
        "marks": [rel(8 + i) for i in range(8)],
    }


def summary(d):
    """Per-op mean microseconds: total, before the first wait, waiting, body, signal."""
    out = {}
    wait = np.nan_to_num(d["wa1"] - d["wa0"]) + np.nan_to_num(d["wb1"] - d["wb0"])
    first_wait = np.where(np.isnan(d["wa0"]), d["wb0"], d["wa0"])
    last_wait_end = np.where(np.isnan(d["wb1"]), d["wa1"], d["wb1"])
    pre = np.where(np.isnan(first_wait), 0.0, first_wait - d["start"])
    body_start = np.where(np.isnan(last_wait_end), d["start"], last_wait_end)
    body = d["body"] - body_start
    sig = d["end"] - d["body"]
    tot = d["end"] - d["start"]
    for op, name in OPS.items():
        m = d["op"] == op
        if not m.any():
            continue
        out[name] = {"n": int(m.sum()), "total": float(np.mean(tot[m])), "pre": float(np.mean(pre[m])),
                     "wait": float(np.mean(wait[m])), "body": float(np.mean(body[m])),
                     "signal": float(np.mean(sig[m])), "sum_total": float(np.sum(tot[m]))}
    span = float(np.nanmax(d["end"]) - np.nanmin(d["start"]))
    busy = float(np.nansum(tot - wait))
    n_cu = int(d["cu"].max()) + 1
    return {"ops": out, "span_us": span, "n_cu": n_cu,
            "busy_frac": busy / (span * n_cu) if span > 0 else 0.0,
            "wait_frac": float(np.nansum(wait)) / (span * n_cu) if span > 0 else 0.0}


def stages(d):
    """(op, layer) -> (first start, last end, first data ready) in us, sorted by first start."""
    keys = {}
    for i in range(len(d["op"])):
        if np.isnan(d["start"][i]):
            continue
        k = (OPS.get(int(d["op"][i]), str(d["op"][i])), int(d["layer"][i]))
        s, e = d["start"][i], d["end"][i]
        r = d["wb1"][i] if not np.isnan(d["wb1"][i]) else (d["wa1"][i] if not np.isnan(d["wa1"][i]) else s)
        if k in keys:
            a, b, c = keys[k]
            keys[k] = (min(a, s), max(b, e), min(c, r))
        else:
            keys[k] = (s, e, r)
    return sorted(keys.items(), key=lambda kv: kv[1][0])


def format_summary(sm):
    lines = [f"step span {sm['span_us']:.1f} us on {sm['n_cu']} CUs; busy {100 * sm['busy_frac']:.1f}%, "
             f"waiting {100 * sm['wait_frac']:.1f}%",
             f"{'op':8s} {'n':>6s} {'total':>8s} {'pre':>8s} {'wait':>8s} {'body':>8s} {'signal':>8s}  (mean us)"]
    for name, v in sm["ops"].items():
        lines.append(f"{name:8s} {v['n']:6d} {v['total']:8.2f} {v['pre']:8.2f} {v['wait']:8.2f} "
                     f"{v['body']:8.2f} {v['signal']:8.2f}")
    return "\n".join(lines)


def layer_timeline(d, layers=None):
    """Per operation of a layer: (median, last) task end in us after the median
    end of the previous layer's last stage (the expert stage at batch 1, the
    expert combine in a batch), averaged over `layers` (default: the middle
    layers); and the per-layer durations (median, min, max)."""
    ops = [int(o) for o in np.unique(d["op"]) if int(o) in OPS]
    batch = 15 in ops
    last_op = 15 if batch else 6
    L = int(d["layer"][d["op"] == last_op].max()) + 1
    if layers is None:
        layers = range(max(1, L // 6), max(2, L - L // 6))
    ends = {l: float(np.median(d["end"][(d["op"] == last_op) & (d["layer"] == l)])) for l in range(L)}
    rows = {}
    for op in ops:
        if op in (8, 9, 16, 17):  # LM head and final task: once per step
            continue
        med, mx = [], []
        for l in layers:
            m = (d["op"] == op) & (d["layer"] == l)
            if l - 1 in ends and m.any():
                med.append(float(np.median(d["end"][m])) - ends[l - 1])
                mx.append(float(np.max(d["end"][m])) - ends[l - 1])
        if med:
            rows[OPS[op]] = (float(np.mean(med)), float(np.mean(mx)), int(((d["op"] == op) & (d["layer"] == layers[0])).sum()))
    per = [ends[l] - ends[l - 1] for l in range(1, L)]
    return rows, (float(np.median(per)), float(min(per)), float(max(per)))
