"""HBM traffic of the megakernel from rocprofv3 byte counters.

Two counter runs of the same bench command, one collecting FETCH_SIZE and
one WRITE_SIZE (KiB per dispatch), each also hold the stream-copy probe's
launches (mk_stream_copy, a known number of bytes read and written). The
copy's reading divided by its known size is the counter's scale on this
device; the megakernel's mean reading divided by that scale is its HBM
traffic per launch. Writes a JSON entry keyed by workload, stamped with the
kernel-source hash, so that the figure is dropped once the kernel changes.

    python -m decode_megakernel_persistent_amd.counters --workload moe48_b1_8k \
        --fetch <run1>/run_counter_collection.csv --write <run2>/run_counter_collection.csv \
        --copy-bytes 1073741824 --out profiles/traffic.json
"""
import argparse
import csv
import json
import os
import statistics


def per_kernel(path, counter):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 CSV."""
    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def pick(d, key):
    names = [k for k in d if key in k]
    if len(names) != 1:
        raise SystemExit(f"expected one kernel matching {key!r}, found {names}")
    return d[names[0]]


def scaled(path, counter, copy_bytes, skip):
    d = per_kernel(path, counter)
    copy_kib = pick(d, "mk_stream_copy_kernel")
    mega_kib = pick(d, "megakernel")[skip:]
    scale = statistics.median(copy_kib) * 1024.0 / copy_bytes
    return {"counter": counter, "copy_kib_median": statistics.median(copy_kib),
            "scale": scale, "kernel_kib_mean": statistics.fmean(mega_kib),
            "dispatches": len(mega_kib),
            "bytes_per_launch": statistics.fmean(mega_kib) * 1024.0 / scale}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--skip", type=int, default=0, help="leading megakernel dispatches to drop")
    ap.add_argument("--command", default="")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    from . import kernel_hash
    fe = scaled(a.fetch, "FETCH_SIZE", a.copy_bytes, a.skip)
    wr = scaled(a.write, "WRITE_SIZE", a.copy_bytes, a.skip)
    entry = {"kernel_hash": kernel_hash(), "fetch": fe, "write": wr,
             "bytes_per_launch": fe["bytes_per_launch"] + wr["bytes_per_launch"],
             "command": a.command}
    data = json.load(open(a.out)) if os.path.exists(a.out) else {}
    data[a.workload] = entry
    with open(a.out, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(entry, indent=1))


if __name__ == "__main__":
    main()
