"""Decode throughput of the persistent megakernel on one GPU.

A step is one decode step of the whole batch (every layer, the LM head and
the greedy argmax) in ONE persistent-kernel launch. Default workload: the
48-layer MoE (hidden 2048, 32/4 heads of 128, 128 experts top-8 of width
768, vocab 151936) at batch 1 with 8192 prior tokens in 16-token pages,
seeded random-init bf16 weights and KV, all resident in HBM before timing.

Prints ONE JSON line: tok/s, ms per step, the megakernel's achieved HBM
bandwidth over the step's algorithmic bytes (weights actually read + KV
read and written) against the 8 TB/s peak, and the CPU oracle timed on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tok/s at batch 1 & 32; achieved HBM GB/s as % of speed-of-light"
HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 30      # stream-copy probe: bytes copied per launch


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="moe48_b1_8k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-steps", type=int, default=3,
                    help="oracle steps in the CPU baseline sample (0: skip)")
    ap.add_argument("--n-cu", type=int, default=0)
    ap.add_argument("--split-pages", type=int, default=0)
    ap.add_argument("--plan-flags", type=int, default=0, help="MK_PLAN_* bits")
    ap.add_argument("--batch32-steps", type=int, default=64,
                    help="timed steps of the batch-32 leg (48-layer MoE at 8K only; 0: skip)")
    ap.add_argument("--sample-steps", type=int, default=64,
                    help="timed steps of the sampling leg (same workload, top-k/top-p/temperature; 0: skip)")
    ap.add_argument("--prefill-steps", type=int, default=16,
                    help="timed 32-token prefill chunks after 8192 prior tokens (48-layer MoE; 0: skip)")
    ap.add_argument("--trace-steps", type=int, default=0,
                    help="after the timed run, this many steps with the per-task trace on (0: none)")
    ap.add_argument("--trace-out", default="", help="markdown file for the traced steps' per-layer timeline")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM counter bytes per launch measured by rocprofv3 --pmc")
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode step runs on a single device "
              "and there is no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import decode_megakernel_persistent_amd as mk

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_gbs = stream_copy_probe(torch, mk, dev)
    r = run_workload(torch, mk, dev, a.workload, a.steps, a.warmup, a)
    w, dec, pool, W = r.pop("w"), r.pop("dec"), r.pop("pool"), r.pop("weights")
    m, B, L = w["model"], w["batch"], w["model"]["n_layers"]
    tok_s, ms_step, per, wall = r["tok_s"], r["ms_step"], r["per"], r["wall"]
    bytes_step, wsum, ksum = r["bytes_step"], r["wsum"], r["ksum"]
    achieved_gbs, sol_tok_s = r["achieved_gbs"], r["sol_tok_s"]
    plan_n_cu, plan_tasks = mk.mk_plan_n_cu(dec.plan), mk.mk_plan_n_tasks(dec.plan)

    traffic = None
    if os.path.exists(a.traffic_json):
        try:
            tj = json.load(open(a.traffic_json))
            ent = tj.get(a.workload)
            if ent and ent.get("kernel_hash") == mk.kernel_hash():
                traffic = ent.get("bytes_per_launch")
        except Exception:
            traffic = None

    cpu = None
    if a.cpu_steps > 0:
        cpu = cpu_baseline(w, a, r["hist"], r["ids"], W)

    # every further leg sets up its own session on the resident weights
    mk.mk_pool_free(pool)
    dec.close()
    dec = pool = None
    torch.cuda.empty_cache()

    if a.trace_steps > 0:
        trace_leg(torch, mk, dev, W, a)
        torch.cuda.empty_cache()

    # sampling beyond greedy in the last stage: the same workload
    smp = None
    if a.sample_steps > 0:
        rs = run_workload(torch, mk, dev, a.workload, a.sample_steps, 2, a, weights=W, sampling=True)
        smp = {"steps": a.sample_steps, "settings": "temperature 0.8, top_k 40, top_p 0.95, min_p 0.05, "
                                                   "one seeded uniform per sequence and step",
               "value": round(rs["tok_s"], 2), "unit": "tok/s", "ms_per_step": round(rs["ms_step"], 4),
               "ms_over_greedy": round(rs["ms_step"] - ms_step, 4)}
        mk.mk_pool_free(rs["pool"])
        rs["dec"].close()
        rs.clear()
        torch.cuda.empty_cache()

    # chunked prefill: 32 prompt tokens of one sequence per step
    pre = None
    if a.prefill_steps > 0 and a.workload == "moe48_b1_8k":
        pre = prefill_leg(torch, mk, dev, W, a)
        torch.cuda.empty_cache()

    # the metric's second number: the same model at batch 32 (ragged contexts,
    # one shared pool), with the weights already resident
    b32 = None
    if a.batch32_steps > 0 and a.workload == "moe48_b1_8k":
        r32 = run_workload(torch, mk, dev, "moe48_b32_ragged", a.batch32_steps, 2, a, weights=W)
        b32 = {"workload": "moe48_b32_ragged", "steps": a.batch32_steps, "warmup": 2,
               "value": round(r32["tok_s"], 2), "unit": "tok/s",
               "ms_per_step": round(r32["ms_step"], 4),
               "context": [min(r32["w"]["ctx"]), max(r32["w"]["ctx"])],
               "bytes_per_step": r32["bytes_step"],
               "achieved_gbs": round(r32["achieved_gbs"], 1),
               "frac": round(r32["achieved_gbs"] / HBM_PEAK_GBS, 4)}
        mk.mk_pool_free(r32["pool"])
        r32["dec"].close()
        r32.clear()

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init bf16 weights N(0,0.02), KV N(0,1), shuffled pages",
        "config": {"workload": a.workload, "batch": B,
                   "context": w["ctx"] if B == 1 else [min(w["ctx"]), max(w["ctx"])],
                   "layers": L, "hidden": m["hidden"], "experts": m["n_experts"],
                   "top_k": m["top_k"], "vocab": m["vocab"], "page_tokens": m["page_tokens"],
                   "n_cu": plan_n_cu, "tasks": plan_tasks},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "bytes_per_step": {"weights": wsum, "kv": ksum, "total": bytes_step},
        "stream_copy": {"gbs": round(copy_gbs, 1), "bytes_per_launch": 2 * COPY_BYTES,
                        "frac_of_copy": round(achieved_gbs / copy_gbs, 4)},
        "sol_tok_s": round(sol_tok_s, 1),
        "frac_of_sol": round(tok_s / sol_tok_s, 4),
        "step_ms": {"median": round(statistics.median(per), 4),
                    "p10": round(sorted(per)[len(per) // 10], 4),
                    "p90": round(sorted(per)[(9 * len(per)) // 10], 4)},
        "host_wall_s": round(wall, 3),
        "cpu_baseline": cpu,
        "batch32": b32,
        "sampling": smp,
        "prefill": pre,
    }
    print(json.dumps(out), flush=True)
    # ordered teardown: plans and pools freed (above), every device buffer
    # released and the device idle before the interpreter (and the HIP
    # runtime with it) shuts down
    del W, r
    torch.cuda.synchronize()
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def run_workload(torch, mk, dev, name, steps, warmup, a, weights=None, sampling=False):
    """Set up workload `name`, run `warmup` steps, restore the starting state,
    time `steps` steps (greedy, or sampled with fixed settings and seeded
    uniform draws) with HIP events on the launch stream, and count the
    algorithmic bytes of every timed step (weights actually read, from the
    step's own top-k ids, plus KV read and written)."""
    from fixtures.session import gpu_session, spec
    w = spec(name, a.seed, steps=warmup + steps)
    m, B = w["model"], w["batch"]
    L = m["n_layers"]
    moe = m["n_experts"] > 0
    K = m["top_k"] if moe else 1
    print(f"[bench] setting up {name}: B={B} ctx={w['ctx'] if B <= 4 else '...'} "
          f"steps={steps} warmup={warmup}", file=sys.stderr, flush=True)
    dec, pool, W = gpu_session(w, a.seed, device=dev, n_cu=a.n_cu, attn_split_pages=a.split_pages,
                               plan_flags=a.plan_flags, weights=weights)
    ctx0 = torch.tensor(w["ctx"], dtype=torch.int32, device=dev)
    tok0 = torch.tensor(w["tokens"], dtype=torch.int32, device=dev)
    # hist[s]: the tokens step s reads; step s writes hist[s + 1]
    hist = torch.empty((max(steps, warmup) + 1, B), dtype=torch.int32, device=dev)
    ids = torch.full((steps, L, B, K), -1, dtype=torch.int32, device=dev)
    smp = [None] * max(steps, warmup)
    if sampling:
        g = torch.Generator().manual_seed(a.seed + 99)
        U = torch.rand((max(steps, warmup), B), generator=g).to(dev)
        base = dict(temperature=torch.full((B,), 0.8, device=dev), top_k=torch.full((B,), 40, dtype=torch.int32, device=dev),
                    top_p=torch.full((B,), 0.95, device=dev), min_p=torch.full((B,), 0.05, device=dev))
        smp = [dict(base, uniform=U[s]) for s in range(max(steps, warmup))]

    # warm-up, then restore the pre-warm-up state (lengths and first tokens)
    hist[0].copy_(tok0)
    for s in range(warmup):
        dec.step(hist[s], hist[s + 1], sampling=smp[s])
    torch.cuda.synchronize()
    dec.check_status()
    dec.seq_lens.copy_(ctx0)
    hist[0].copy_(tok0)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for s in range(steps):
        dec.step(hist[s], hist[s + 1], topk_ids=ids[s] if moe else None, sampling=smp[s])
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec.check_status()
    per = [ev[s].elapsed_time(ev[s + 1]) for s in range(steps)]
    ms_total = ev[0].elapsed_time(ev[steps])

    ids_h = ids.cpu() if moe else None
    desc = mk.model_desc(m)
    tot_bytes = wsum = ksum = 0.0
    for s in range(steps):
        lens = [c + s for c in w["ctx"]]
        distinct = [len(set(ids_h[s, l].reshape(-1).tolist())) for l in range(L)] if moe else None
        wb, kr, kw = mk.mk_step_bytes(desc, lens, distinct)
        tot_bytes += wb + kr + kw
        wsum += wb
        ksum += kr + kw
    bytes_step = tot_bytes / steps
    return {"w": w, "dec": dec, "pool": pool, "weights": W, "hist": hist[:steps + 1].cpu().tolist(),
            "ids": ids_h,
            "tok_s": B * steps / (ms_total * 1e-3), "ms_step": ms_total / steps, "per": per,
            "wall": wall, "bytes_step": bytes_step, "wsum": wsum / steps, "ksum": ksum / steps,
            "achieved_gbs": tot_bytes / (ms_total * 1e-3) / 1e9,
            "sol_tok_s": B * HBM_PEAK_GBS * 1e9 / bytes_step}


def prefill_leg(torch, mk, dev, W, a, C=32, p0=8192):
    """Chunked prefill of the 48-layer MoE: one sequence with p0 prior tokens
    runs C-token chunks (MK_PLAN_PREFILL: C batch rows at consecutive
    positions sharing one page row); each timed step is one chunk, the next
    step the next C positions. Bytes per step are those this design reads:
    the weights the chunk's routing touches and, per row, the K/V of every
    token before it (each row streams the prior context)."""
    from decode_megakernel_persistent_amd.runtime import Decoder, alloc_kv_pool
    from fixtures import device as fxd
    from fixtures.session import spec
    m = spec("moe48_b1_8k", a.seed)["model"]
    L, V, K, pt = m["n_layers"], m["vocab"], m["top_k"], m["page_tokens"]
    warm, steps = 2, a.prefill_steps
    total = p0 + C * (warm + steps + 1)  # the last chunk's last row reads up to its own bound
    n_pages = -(-total // pt)
    pool = mk.mk_pool_create(n_pages, pt, 1, None)
    mk.mk_pool_lease(pool, 0, total)
    row = mk.mk_pool_page_table(pool, [0], n_pages)[0]
    kv = alloc_kv_pool(m, n_pages, dev)
    fxd.fill_kv(kv, torch.tensor(row, dtype=torch.int32, device=dev), m, a.seed, 0, p0)
    lens = [p0 + i for i in range(C)]
    bounds = [x + C * (warm + steps) for x in lens]
    print(f"[bench] prefill: {C}-token chunks after {p0} tokens, {steps} timed", file=sys.stderr, flush=True)
    dec = Decoder(m, W, kv, n_pages, lens, [row] * C, n_pages, max(bounds), device=dev,
                  plan_flags=mk.MK_PLAN_PREFILL, ctx_bounds=bounds)
    g = torch.Generator().manual_seed(a.seed + 5)
    toks = torch.randint(0, V, (warm + steps, C), generator=g, dtype=torch.int32).to(dev)
    out = torch.empty((warm + steps, C), dtype=torch.int32, device=dev)
    ids = torch.full((steps, L, C, K), -1, dtype=torch.int32, device=dev)
    for s in range(warm):
        dec.step(toks[s], out[s])
    torch.cuda.synchronize()
    dec.check_status()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(steps):
        dec.step(toks[warm + s], out[warm + s], topk_ids=ids[s])
    e1.record(stream)
    torch.cuda.synchronize()
    dec.check_status()
    ms = e0.elapsed_time(e1) / steps
    ids_h = ids.cpu()
    desc = mk.model_desc(m)
    tot = 0.0
    for s in range(steps):
        ln = [x + C * (warm + s) for x in lens]
        distinct = [len(set(ids_h[s, l].reshape(-1).tolist())) for l in range(L)]
        wb, kr, kw = mk.mk_step_bytes(desc, ln, distinct)
        tot += wb + kr + kw
    bytes_step = tot / steps
    dec.close()
    mk.mk_pool_free(pool)
    del kv
    gbs = bytes_step / (ms * 1e-3) / 1e9
    return {"chunk": C, "prior_tokens": p0, "steps": steps, "value": round(C / (ms * 1e-3), 1),
            "unit": "prompt tok/s", "ms_per_chunk": round(ms, 4), "bytes_per_chunk": bytes_step,
            "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def stream_copy_probe(torch, mk, dev, reps=5):
    """Achievable streaming bandwidth: mk_stream_copy of COPY_BYTES (read and
    written once each) timed with HIP events on the launch stream. The same
    launches are the known-size kernel that calibrates rocprofv3 byte counters."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        mk.mk_stream_copy(dst.data_ptr(), src.data_ptr(), COPY_BYTES, stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        mk.mk_stream_copy(dst.data_ptr(), src.data_ptr(), COPY_BYTES, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def trace_leg(torch, mk, dev, W, a):
    """a.trace_steps steps of the same workload with the per-task trace on
    (outside the timed run: the trace adds stores to every task); the last
    step's per-layer timeline goes to stderr and, with --trace-out, to a
    markdown file."""
    from decode_megakernel_persistent_amd import trace as T
    from fixtures.session import gpu_session, spec
    # the plan of the timed run (its context bound), traced over its first steps
    w = spec(a.workload, a.seed, steps=max(a.warmup + a.steps, 2 + a.trace_steps))
    B = w["batch"]
    dec, pool, _ = gpu_session(w, a.seed, device=dev, n_cu=a.n_cu, attn_split_pages=a.split_pages,
                               plan_flags=a.plan_flags, weights=W, trace=True)
    hist = torch.empty((3 + a.trace_steps, B), dtype=torch.int32, device=dev)
    hist[0].copy_(torch.tensor(w["tokens"], dtype=torch.int32, device=dev))
    for s in range(2 + a.trace_steps):
        dec.step(hist[s], hist[s + 1])
    torch.cuda.synchronize()
    dec.check_status()
    d = T.decode(dec.trace)
    rows, (pmed, pmin, pmax) = T.layer_timeline(d)
    lines = [f"per-task trace of the last of {2 + a.trace_steps} steps of `{a.workload}`",
             "", "    " + T.format_summary(T.summary(d)).replace("\n", "\n    "), "",
             f"per layer: median {pmed:.2f} us (min {pmin:.2f}, max {pmax:.2f})", "",
             "| stage | tasks per layer | median end (us) | last end (us) |", "|---|---|---|---|"]
    for name, (med, mx, n) in sorted(rows.items(), key=lambda kv: kv[1][0]):
        lines.append(f"| {name} | {n} | {med:.2f} | {mx:.2f} |")
    text = "\n".join(lines)
    print(text, file=sys.stderr, flush=True)
    if a.trace_out:
        with open(a.trace_out, "w") as f:
            f.write(text + "\n")
    mk.mk_pool_free(pool)
    dec.close()


def host_description():
    """nproc, the cores this process may run on, the CPU model and host RAM."""
    info = {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu"] = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                info["ram_gib"] = round(int(line.split()[1]) / 2 ** 20, 1)
                break
    except OSError:
        pass
    return info


def cpu_baseline(w, a, hist, ids, Wd):
    """The oracle on the host cores, on a bounded sample of the same workload,
    teacher-forced on the GPU's run.

    Sample: the first a.cpu_steps timed steps. Step s takes the GPU's input
    tokens of that step (and its routing where the oracle's own top-k is a
    near-tie) and its argmax is compared with the GPU's output token. The
    weights a step touches are copied to host memory before it is timed (from
    the device tensors the fixture generator filled); the KV is the oracle's
    own contiguous copy, drawn by the host generator.
    """
    import torch
    import oracle as O
    from fixtures.hostmodel import DeviceCopyWeights
    from fixtures.session import oracle_inputs
    m = w["model"]
    B, L = w["batch"], m["n_layers"]
    moe = m["n_experts"] > 0
    n = min(a.cpu_steps, len(hist) - 1)
    Wh = DeviceCopyWeights(m, Wd, a.seed)
    _, kv = oracle_inputs(dict(w, steps=n), a.seed, cache=False)
    times, agree, forced_n, differ_n = [], 0, 0, 0
    for s in range(n):
        routing = [[[int(v) for v in ids[s, l, b]] for l in range(L)] for b in range(B)] if moe else None
        for l in range(L):  # the weights this step reads, resident before the timed region
            Wh.wqkv(l), Wh.wo(l)
            if moe:
                Wh.router(l)
                for e in {int(v) for v in ids[s, l].reshape(-1).tolist()}:
                    Wh.gate(l, e), Wh.up(l, e), Wh.down(l, e)
            else:
                Wh.gate(l), Wh.up(l), Wh.down(l)
        Wh.lm_head()
        t0 = time.perf_counter()
        r, forced, differ = O.decode_step_following(m, Wh, kv, hist[s], routing, 1e-3)
        times.append(time.perf_counter() - t0)
        forced_n += len(forced)
        differ_n += len(differ)
        agree += sum(1 for b in range(B) if r["next"][b] == hist[s + 1][b])
        if sum(times) > 60:
            break
    dt = sum(times) / len(times)
    host = host_description()
    return {"value": round(B / dt, 4), "unit": "tok/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"{len(times)} decode step(s) of {a.workload}: the first timed steps, teacher-forced "
                      f"on the GPU's input tokens; weights resident in host memory before timing; "
                      f"mean {dt:.3f} s per step",
            "agreement": f"{agree}/{len(times) * B} next tokens equal the GPU's",
            "routing_near_ties_followed": forced_n, "routing_differences": differ_n,
            "host": host}


if __name__ == "__main__":
    main()
