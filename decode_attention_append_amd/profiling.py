"""Summaries of rocprofv3 output for the committed profiles.

    python -m decode_attention_append_amd.profiling trace  <kernel_stats.csv> <out.md> <title> <command>
    python -m decode_attention_append_amd.profiling counters <fetch_dir> <write_dir> <kernel> <source> <workload>
                                                         <bytes_per_launch> <out.json> <fetch_cmd> <write_cmd>

`counters` reads two rocprofv3 --pmc runs of `bench.py --calibrate-copy` (one with
FETCH_SIZE, one with WRITE_SIZE), takes the average per dispatch of the named kernel,
and scales both by what the same counter reads for the plain 1 GiB device copy the
bench runs first (the three largest copy-kernel dispatches), so the result is HBM
bytes per launch.  It records a hash of the kernel's sources (comments and
whitespace aside), so a later change to the kernel makes the numbers stale
(bench.py then reports traffic as null).
"""
import csv
import glob
import hashlib
import json
import os
import re
import sys

COPY_BYTES = 1 << 30
HERE = os.path.dirname(os.path.abspath(__file__))


def code_text(text: str) -> str:
    """The source without comments and with whitespace runs collapsed: what the
    compiler sees, so that editing a comment does not mark the counters stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(source: str) -> str:
    h = hashlib.sha256()
    for name in (source, "da_internal.h"):
        with open(os.path.join(HERE, "csrc", name)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def _per_dispatch(run_dir: str, counter: str):
    """{dispatch_id: (kernel_name, value)} summed over counter dimensions."""
    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            key = (path, row["Dispatch_Id"])
            name, v = out.get(key, (row["Kernel_Name"], 0.0))
            out[key] = (name, v + float(row["Counter_Value"]))
    return list(out.values())


def _kernel_avg(rows, kernel: str):
    vals = [v for name, v in rows if kernel in name]
    if len(vals) > 1:
        vals = vals[1:]  # the first launch also pays code and table warm-up
    return sum(vals) / len(vals) if vals else None, len(vals)


def _copy_avg(rows):
    vals = sorted((v for name, v in rows if "copy" in name.lower()), reverse=True)[:3]
    return sum(vals) / len(vals) if vals else None


def counters(fetch_dir, write_dir, kernel, source, workload, bytes_per_launch, out_json, fetch_cmd,
             write_cmd):
    fr, wr = _per_dispatch(fetch_dir, "FETCH_SIZE"), _per_dispatch(write_dir, "WRITE_SIZE")
    fetch_kib, n_f = _kernel_avg(fr, kernel)
    write_kib, n_w = _kernel_avg(wr, kernel)
    copy_fetch, copy_write = _copy_avg(fr), _copy_avg(wr)
    f_scale = (COPY_BYTES / 1024) / copy_fetch
    w_scale = (COPY_BYTES / 1024) / copy_write
    hbm = (fetch_kib * f_scale + write_kib * w_scale) * 1024
    rec = {
        "kernel": kernel, "workload": workload, "source": source,
        "source_sha256": source_hash(source),
        "fetch_kib_per_dispatch": round(fetch_kib, 1), "write_kib_per_dispatch": round(write_kib, 1),
        "dispatches": [n_f, n_w],
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": round(copy_fetch, 1),
                             "write_kib": round(copy_write, 1), "fetch_scale": round(f_scale, 4),
                             "write_scale": round(w_scale, 4)},
        "hbm_bytes_per_launch": int(hbm),
        "algorithmic_bytes_per_launch": int(bytes_per_launch),
        "traffic_over_algorithmic": round(hbm / float(bytes_per_launch), 4),
        "commands": [fetch_cmd, write_cmd],
    }
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def trace(stats_csv, out_md, title, command):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# Kernel trace: {title}", "", "Command (from the repository root on an MI355X, rocprofv3 of ROCm 7.2):",
             "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        n = n if len(n) <= 70 else n[:67] + "..."
        lines.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:6])
    elif sys.argv[1] == "counters":
        a = sys.argv[2:]
        print(json.dumps(counters(a[0], a[1], a[2], a[3], a[4], int(a[5]), a[6], a[7], a[8]), indent=1))
