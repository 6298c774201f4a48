"""Summaries of rocprofv3 output for the committed profiles.

    python -m decode_attention_append_amd.profiling trace  <run_dir> <out.md> <title> <command> [<warm_launches>]
    python -m decode_attention_append_amd.profiling counters <fetch_dir> <write_dir> <kernel> <source> <workload>
                                                         <bytes_per_launch> <out.json> <fetch_cmd> <write_cmd>

`counters` reads two rocprofv3 --pmc runs of `bench.py --calibrate-copy` (one with
FETCH_SIZE, one with WRITE_SIZE), takes the average per dispatch of the named kernel,
and scales both by what the same counter reads for the plain 1 GiB device copy the
bench runs first (the three largest copy-kernel dispatches), so the result is HBM
bytes per launch.  It records a hash of the kernel's sources (comments and
whitespace aside), so a later change to the kernel makes the numbers stale
(bench.py then reports traffic as null).

`trace` reads the per-dispatch kernel trace of a `rocprofv3 --kernel-trace` run
of bench.py and reports, per kernel, all launches and the cold ones only: when
the run read the 2 GiB cache-flush buffer before its timed steps, the launches
after the first flush; otherwise every launch after the first `warm_launches`
(the warm-up steps), which then stream more than the caches hold anyway.
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


def _launches(run_dir):
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]


def _is_flush(name):
    return "reduce_kernel" in name


def _is_ours(name):
    return re.match(r"(void )?da::", name) is not None


def _stats(v):
    v = sorted(v)
    return len(v), sum(v) / len(v), v[len(v) // 2], v[0], v[-1]


def trace(run_dir, out_md, title, command, warm_launches=0):
    launches = _launches(run_dir)
    ours = [n for n, _ in launches if _is_ours(n)]
    flushed = any(_is_flush(n) for n, _ in launches)
    cold, seen_flush, per_kernel_seen = {}, False, {}
    for n, us in launches:
        if _is_flush(n):
            seen_flush = True
            continue
        if not _is_ours(n):
            continue
        per_kernel_seen[n] = per_kernel_seen.get(n, 0) + 1
        if (flushed and seen_flush) or (not flushed and per_kernel_seen[n] > warm_launches):
            cold.setdefault(n, []).append(us)
    rule = ("launches after the first read of the 2 GiB cache-flush buffer (every timed step is preceded by one)"
            if flushed else f"every launch after the first {warm_launches} of each kernel (the warm-up steps); "
            "each step streams more than the caches hold")
    lines = [f"# Kernel trace: {title}", "", "Command (from the repository root on an MI355X, rocprofv3 of ROCm 7.2):",
             "", "```", command, "```", "",
             f"Cold launches: {rule}.", "",
             "| kernel | cold launches | cold mean us | cold median us | cold min us | cold max us | all launches | all mean us |",
             "|---|---|---|---|---|---|---|---|"]
    for n in sorted(set(ours), key=ours.index):
        allv = [us for k, us in launches if k == n]
        short = n if len(n) <= 70 else n[:67] + "..."
        if n in cold:
            c, mean, med, lo, hi = _stats(cold[n])
            lines.append(f"| `{short}` | {c} | {mean:.2f} | {med:.2f} | {lo:.2f} | {hi:.2f} | {len(allv)} | "
                         f"{sum(allv) / len(allv):.2f} |")
        else:
            lines.append(f"| `{short}` | 0 | - | - | - | - | {len(allv)} | {sum(allv) / len(allv):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return {n: _stats(v) for n, v in cold.items()}


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:6], *(int(x) for x in sys.argv[6:7]))
    elif sys.argv[1] == "counters":
        a = sys.argv[2:]
        print(json.dumps(counters(a[0], a[1], a[2], a[3], a[4], int(a[5]), a[6], a[7], a[8]), indent=1))
