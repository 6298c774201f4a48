#!/usr/bin/env python3
"""Throughput of one decode step of GQA attention with KV append on one MI355X.

A step is the whole path over one batch: for every layer, the KV append, the
split-context attention and the combine, enqueued on one stream.  By default
each layer is one da_decode_step call (append and merge fused into the
attention launch where the plan allows); --path separate times the three
separate calls da_kv_append, da_gqa_decode_attn, da_gqa_decode_attn_combine.
The default workload is batched GQA decode with Hq 16 / Hkv 8 / head_dim 128,
batch 32, context 8192, 28 layers (bf16, synthetic N(0,1)*0.5 inputs resident
in HBM before timing starts).

One whole step (every layer) is captured into a HIP graph once, after the
warm-up steps, and a multi-layer step is timed as its replays: each replay runs
every layer's kernels on the same inputs, exactly as an eager step does (the
graph tests check replays against eager steps bit for bit), without the host
launch gaps between layers.  The same step is also timed as eager launches, which
start sooner on the GPU than a graph, and each record carries both figures and
the host's time to enqueue an eager step; the step's figure is the faster where
the host keeps up.  --eager times eagerly launched steps only, with no capture.  Steps that
touch less than 1 GiB start cold: a 2 GiB buffer is read before each of them,
outside the timing.

Prints ONE JSON line: KV GB/s (algorithmic bytes per step / step time), ms per
step, the attention kernel's roofline fraction against the 8 TB/s HBM peak, the
fp64 CPU oracle's rate on a bounded sample of the same workload, and under
"configs" the same measurements for every other workload of the suite (the
512-context layer, the MHA 4k layers, GQA-8 long context, the 4-token verify,
the head_dim-256 gated layers), each measured in a child process of its own
(as the workload would run alone).  Each record also carries the attention
kernel's mean duration over cold launches, read from the GPU's own kernel
timestamps (torch's profiler), and its fraction of the HBM peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path step|separate]
                    [--eager] [--configs all|none] [--no-cpu-baseline] [--no-kernel-profiler]
"""
import argparse
import json
import os
import subprocess
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first tenth of a second or so of sustained load runs up to 5% slow (the
    # default workload's first 5-20 steps in a process take 4.6 ms, the rest 4.4 ms):
    # the default warm-up covers it
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--chunk", type=int, default=0, help="chunk_tokens override (0 = automatic)")
    ap.add_argument("--items", type=int, default=0,
                    help="balanced chunking: chunks to aim for over the launch (0 = the library's default)")
    ap.add_argument("--path", choices=["step", "separate"], default="step",
                    help="step: one da_decode_step per layer; separate: the three calls per layer")
    ap.add_argument("--rope", type=float, default=0.0, metavar="THETA",
                    help="fuse the rotary embedding with this base (e.g. 1e6): the append rotates new K "
                         "rows and the attention rotates q")
    ap.add_argument("--paged", action="store_true",
                    help="paged caches: every layer's K/V cache becomes a pool of 16-token pages in a "
                         "random order behind one block table")
    ap.add_argument("--eager", action="store_true",
                    help="time eagerly launched steps instead of replays of the step captured into a HIP "
                         "graph")
    ap.add_argument("--configs", choices=["all", "none"], default=None,
                    help="also measure every other workload of the suite (default: all for the default "
                         "workload, none when --workload is given)")
    ap.add_argument("--config-steps", type=int, default=100, help="timed steps per extra workload")
    ap.add_argument("--config-record", action="store_true",
                    help="print only the per-workload record that the default run collects under "
                         "\"configs\" (what the default run starts once per workload, in a process of its own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-profiler", action="store_true",
                    help="skip the kernel durations from torch's profiler (e.g. under rocprofv3)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--flush", choices=["auto", "on", "off"], default="auto",
                    help="read a 2 GiB buffer before every timed step (outside the timed span) so the "
                         "step starts with cold caches; auto = on when one step touches less than "
                         "1 GiB, which the 256 MB Infinity Cache could otherwise serve")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy three times, so that hardware "
                         "byte counters can be scaled by a kernel of known traffic")
    return ap.parse_args()


def algorithmic_bytes(w, seq_pos):
    """Bytes the step must move at least, per layer: K+V of the visible context read once,
    q read, out written (and the output gate read, when gated), new K/V read and written
    into the cache."""
    E, D = 2, w.head_dim
    ctx = [int(s) + w.q_len for s in seq_pos]
    kv = 2 * w.n_kv_heads * sum(ctx) * D * E
    q_out = (3 if w.gated else 2) * w.batch * w.q_len * w.n_q_heads * D * E
    append = 2 * 2 * w.batch * w.q_len * w.n_kv_heads * D * E
    return kv, kv + q_out + append


def counters_for(kernel_tag, workload):
    """HBM bytes per launch of the kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), if it was taken
    on the current kernel sources; else None."""
    from decode_attention_append_amd import profiling
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"counters_{kernel_tag}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    try:
        if profiling.source_hash(rec["source"]) != rec.get("source_sha256"):
            return None
    except (KeyError, OSError):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, layers_host_fn, n_layers, budget_s, freqs=None, block_table=None):
    """The oracle (append + attention, fp64, OpenMP; with the rotary embedding when a
    table is given, the output gate when the workload has one) on whole layers of the
    workload until about budget_s of CPU time is spent; returns the record for the JSON
    line."""
    import oracle
    dt = oracle.FP16 if w.dtype == "fp16" else oracle.BF16
    import numpy as np
    done_bytes, spent, n = 0, 0.0, 0
    for layer in range(n_layers):
        q, kc, vc, kn, vn, sp, gate = layers_host_fn(layer)
        t = time.perf_counter()
        if freqs is not None:
            pos = sp[:, None, None] + np.arange(w.q_len, dtype=np.int32)[None, :, None]
            kn = oracle.rope_rows(kn, np.broadcast_to(pos, kn.shape[:3]), freqs, dt)
            q = oracle.rope_q(q, sp, freqs, dt)
        if block_table is None:
            k2, v2 = oracle.kv_append(kc, vc, kn, vn, sp)
        else:
            kp, vp = oracle.kv_append_paged(kc, vc, kn, vn, sp, block_table)
            k2, v2 = oracle.gather_paged(kp, block_table), oracle.gather_paged(vp, block_table)
        out = oracle.gqa_decode(q, k2, v2, sp, dt)
        if gate is not None:
            oracle.output_gate(out, gate, dt)
        spent += time.perf_counter() - t
        done_bytes += algorithmic_bytes(w, sp)[1]
        n += 1
        del k2, v2, kc, vc
        if spent >= budget_s:
            break
    return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} of {w.layers} layers of {w.name}, every sequence and head, "
                      f"append + attention in fp64 ({spent:.1f} s)"}


class Bench:
    """One workload on the GPU: its layers, problems, workspace and step functions."""

    def __init__(self, w, args, dev, path, theta=0.0, paged=False, chunk=0, items=0):
        import torch
        import decode_attention_append_amd as da
        from decode_attention_append_amd.workloads import make_layer, rope_freqs
        self.w, self.dev, self.path, self.paged = w, dev, path, paged
        self.layers = [make_layer(w, l, dev) for l in range(w.layers)]
        self.seq_pos = self.layers[0]["seq_pos"].cpu().numpy()
        self.theta = theta if theta > 0 else w.rope_theta
        self.rope_dim = w.rope_dim or w.head_dim
        self.freqs = rope_freqs(self.rope_dim, self.theta, dev) if self.theta > 0 else None
        self.block_table, n_pages = None, 0
        if paged:
            # pages of every (sequence, KV head) cache, shuffled into one pool per layer and cache
            pps = w.max_seq // 16
            n_pages = w.batch * pps
            perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(7))
            self.block_table = perm.view(w.batch, pps).to(torch.int32).to(dev)
            inv = torch.empty_like(perm)
            inv[perm] = torch.arange(n_pages)
            for L in self.layers:
                for key in ("k_cache", "v_cache"):
                    c = L[key].view(w.batch, w.n_kv_heads, pps, 16, w.head_dim).transpose(1, 2)
                    pages = c.reshape(n_pages, w.n_kv_heads, 16, w.head_dim)  # page b * pps + i
                    L[key] = pages[inv.to(dev)].contiguous()  # pool page perm[j] holds page j
                    del c, pages
            torch.cuda.synchronize()
        # one problem per layer: a gated problem carries its layer's gate tensor
        self.probs = [da.problem(w.batch, w.q_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_seq, w.dtype,
                                 chunk_tokens=chunk, work_items=items, rope_freqs=self.freqs,
                                 block_table=self.block_table, n_pages=n_pages,
                                 rope_dim=self.rope_dim if self.freqs is not None else 0,
                                 out_gate=L.get("out_gate"))
                      for L in self.layers]
        self.plan = da.plan_attention(self.probs[0])
        self.ws = da.new_workspace(self.probs[0])
        self.outs = [torch.empty_like(L["q"]) for L in self.layers]
        self.stream = torch.cuda.current_stream()
        self.launch_stream = [self.stream]  # None while capturing: the binding then uses torch's stream
        self.da = da
        torch.cuda.synchronize()

    def step(self, events=None):
        da, s = self.da, self.launch_stream[0]
        for l, L in enumerate(self.layers):
            p = self.probs[l]
            if self.path == "separate":
                da.kv_append(p, L["k_cache"], L["v_cache"], L["k_new"], L["v_new"], L["seq_pos"], s)
                if events is not None:
                    events[l][0].record(self.stream)
                da.gqa_decode_attn(p, L["q"], L["k_cache"], L["v_cache"], L["seq_pos"], self.ws, s)
                if events is not None:
                    events[l][1].record(self.stream)
                da.gqa_decode_attn_combine(p, self.ws, L["seq_pos"], self.outs[l], s)
            else:
                if events is not None:
                    events[l][0].record(self.stream)
                da.decode_step(p, L["q"], L["k_cache"], L["v_cache"], L["k_new"], L["v_new"], L["seq_pos"],
                               self.ws, self.outs[l], s)
                if events is not None:
                    events[l][1].record(self.stream)

    def kernel_name(self):
        w = self.w
        kernel = "attn_split_" + self.plan["variant"] + ("256" if w.head_dim == 256 else "")
        if self.paged:
            kernel += "_paged"
        if self.freqs is not None:
            kernel += "_rope"
        if w.gated:
            kernel += "_gate"
        return kernel

    def bytes(self):
        """(algorithmic bytes per step, per attention launch)."""
        w = self.w
        kv_bytes, alg_bytes = algorithmic_bytes(w, self.seq_pos)
        # The attention launch reads the K+V of the visible context (512 bytes per
        # visible key per KV head at head_dim 128) and q; in the one-launch step it
        # also writes the new rows into the cache and, with the merge fused, the
        # output (reading the gate).  There the new rows are read once, from k_new,
        # as part of the visible context.
        q_bytes = w.batch * w.q_len * w.n_q_heads * w.head_dim * 2
        attn_bytes = kv_bytes + q_bytes
        if self.path == "step":
            attn_bytes += 2 * w.batch * w.q_len * w.n_kv_heads * w.head_dim * 2
            if self.plan["fused_combine"]:
                attn_bytes += q_bytes * (2 if w.gated else 1)
        return alg_bytes * w.layers, attn_bytes

    def measure(self, steps, warmup, eager, flush_mode, kernel_profiler):
        """Timed steps (graph replays and eager launches, or eager launches only),
        HIP events around every attention launch of an eager pass, and optionally the attention kernels' durations from
        the profiler over cold launches."""
        import numpy as np
        import torch
        w = self.w
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        step_bytes, attn_bytes = self.bytes()
        flush = flush_mode == "on" or (flush_mode == "auto" and step_bytes < (1 << 30))
        flush_buf = torch.ones(1 << 30, dtype=torch.bfloat16, device=self.dev) if flush else None
        ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(w.layers)] for _ in range(steps)]
        # one event pair per step (back to back when there is no flush), so the
        # spread of the step time is reported beside its mean
        marks = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                 for _ in range(steps)]
        torch.cuda.synchronize()
        step_ms = []

        def timed(run, host_s=None):
            for k in range(steps):
                if flush:
                    flush_buf.sum(dtype=torch.float32)  # outside the timed span of the step
                marks[k][0].record(self.stream)
                t0 = time.perf_counter()
                run(k)
                if host_s is not None:
                    host_s.append(time.perf_counter() - t0)
                marks[k][1].record(self.stream)
            torch.cuda.synchronize()
            step_ms[:] = [a.elapsed_time(b) for a, b in marks]
            return sum(step_ms)

        ms_graph = ms_eager = None
        if not eager:
            graph = torch.cuda.CUDAGraph()
            self.launch_stream[0] = None
            with torch.cuda.graph(graph):
                self.step()
            self.launch_stream[0] = self.stream
            torch.cuda.synchronize()
            # W more untimed replays before the timed ones, for the same settling
            for _ in range(max(1, warmup)):
                graph.replay()
            torch.cuda.synchronize()
            ms_graph = timed(lambda k: graph.replay())
            graph_ms = list(step_ms)
            host_s = []
            ms_eager = timed(lambda k: self.step(), host_s)
            eager_ms = list(step_ms)
            host_ms = float(np.mean(host_s)) * 1e3
            timed(lambda k: self.step(ev[k]))  # eager pass for the kernel's own duration
            # Both timings go into the record, and the step's figure is the faster
            # of the two where the host enqueued an eager step in no more time than
            # the GPU ran it (so that it holds in a loop with no head start).  A
            # graph launch costs more on the GPU's timeline than eager launches
            # (about 14 us from event to event for a graph of one tiny kernel,
            # against 6.5 us for the kernel launched eagerly); a graph removes the
            # host's launch gaps where the host enqueues slower than the GPU runs.
            if ms_eager < ms_graph and host_ms * steps <= ms_eager:
                timing, ms_total, step_ms[:] = "eager", ms_eager, eager_ms
            else:
                timing, ms_total, step_ms[:] = "graph", ms_graph, graph_ms
            del graph
        else:
            timing, host_ms = "eager", None
            ms_total = timed(lambda k: self.step(ev[k]))
        attn_ms = [e0.elapsed_time(e1) for evk in ev for (e0, e1) in evk]

        kernel_us = None
        if kernel_profiler:
            from torch.profiler import ProfilerActivity, profile
            n_prof = max(5, min(steps, 20))
            with profile(activities=[ProfilerActivity.CUDA]) as prof:
                for _ in range(n_prof + 1):
                    if flush:
                        flush_buf.sum(dtype=torch.float32)
                    self.step()
                torch.cuda.synchronize()
            kernel_us = {}
            for e in sorted(prof.events(), key=lambda e: e.time_range.start):
                for tag in ("attn_split", "attn_combine", "kv_append"):
                    if tag in e.name:
                        kernel_us.setdefault(tag, []).append(float(e.device_time))
            # the first profiled step's launches also pay the profiler's own start-up
            kernel_us = {t: v[w.layers:] for t, v in kernel_us.items() if len(v) > w.layers}
        del flush_buf
        return {"ms_total": ms_total, "step_ms": step_ms, "attn_ms": attn_ms, "flush": flush,
                "step_bytes": step_bytes, "attn_bytes": attn_bytes, "kernel_us": kernel_us,
                "timing": timing, "ms_graph": ms_graph, "ms_eager": ms_eager, "host_ms": host_ms}


def both_timings(m, steps):
    """us per step by graph replay and by eager launches, where both were timed."""
    if m["ms_graph"] is None:
        return {}
    return {"us_per_step_graph": round(m["ms_graph"] / steps * 1e3, 2),
            "us_per_step_eager": round(m["ms_eager"] / steps * 1e3, 2),
            "host_us_per_eager_step": round(m["host_ms"] * 1e3, 2)}


def config_record(b, m, steps):
    """The JSON record of one workload's measurements (see the module docstring)."""
    import numpy as np
    w, plan = b.w, b.plan
    ms = m["ms_total"] / steps
    rec = {
        "us_per_step": round(ms * 1e3, 2),
        "us_per_step_p10_p50_p90": [round(float(np.percentile(m["step_ms"], q)) * 1e3, 2) for q in (10, 50, 90)],
        "gbs": round(m["step_bytes"] / (ms * 1e-3) / 1e9, 2),
        "hbm_frac": round(m["step_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_step": m["step_bytes"],
        "kernel": b.kernel_name(),
        "kernel_bytes_per_launch": m["attn_bytes"],
        "variant": plan["variant"], "path": b.path,
        "fused_merge": bool(plan["fused_combine"]) and b.path == "step",
        "launches_per_layer": (3 if b.path == "separate" else (1 if plan["fused_combine"] else 2)),
        "layers": w.layers, "graph": m["timing"] == "graph", **both_timings(m, steps),
        "cold_cache_flush": m["flush"], "context": int(b.seq_pos.max()) + w.q_len,
    }
    ku = m["kernel_us"]
    if ku and ku.get("attn_split"):
        us = float(np.mean(ku["attn_split"]))
        rec["kernel_us_profiler"] = round(us, 2)
        rec["kernel_gbs"] = round(m["attn_bytes"] / (us * 1e-6) / 1e9, 2)
        rec["kernel_frac"] = round(m["attn_bytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        rec["kernel_launches_profiled"] = len(ku["attn_split"])
        if ku.get("attn_combine"):
            rec["combine_us_profiler"] = round(float(np.mean(ku["attn_combine"])), 2)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the step shards by sequence or KV head with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decode_attention_append_amd.workloads import BENCH_WORKLOAD, WORKLOADS

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    configs = args.configs or ("none" if args.workload else "all")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] workload {w.name}: building {w.layers} layers on {torch.cuda.get_device_name(0)}",
          file=sys.stderr, flush=True)

    b = Bench(w, args, dev, args.path, args.rope, args.paged, args.chunk, args.items)
    m = b.measure(args.steps, args.warmup, args.eager, args.flush, not args.no_kernel_profiler)
    if args.config_record:
        print(json.dumps(config_record(b, m, args.steps)), flush=True)
        return
    ms_per_step = m["ms_total"] / args.steps
    step_bytes, attn_bytes = m["step_bytes"], m["attn_bytes"]
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: the split-context attention.  Its duration from the HIP events
    # around every launch, bounded by the step time per layer (with one launch per
    # layer), which the events can only exceed by their own overhead.
    attn_ms = m["attn_ms"]
    attn_avg_ms = float(np.mean(attn_ms))
    if args.path == "step" and b.plan["fused_combine"]:
        attn_avg_ms = min(attn_avg_ms, ms_per_step / w.layers)
    kernel = b.kernel_name()
    kernel_tag = kernel
    if args.path == "step":
        kernel_tag += "_step" if b.plan["fused_combine"] else "_step+attn_combine"
    attn_gbs = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    # counters of the attention launch (the dominant kernel, whose bytes `achieved` uses)
    traffic = counters_for(kernel_tag.split("+")[0], w.name)

    rec = {
        "metric": "decode-attention KV GB/s (% of HBM peak) + us/step, Hq16/Hkv8/d128 ctx 8k",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_p10_p50_p90": [round(float(np.percentile(m["step_ms"], q)) * 1e3, 2) for q in (10, 50, 90)],
        **both_timings(m, args.steps),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "context": int(b.seq_pos.max()) + w.q_len,
                   "max_seq": w.max_seq, "layers": w.layers, "chunk_tokens": b.plan["chunk_tokens"],
                   "target_items": b.plan["target_items"],
                   "variant": b.plan["variant"], "path": args.path, "graph": m["timing"] == "graph",
                   "rope_theta": b.theta if b.freqs is not None else None,
                   "rope_dim": b.rope_dim if b.freqs is not None else None, "output_gate": w.gated,
                   "paged": args.paged,
                   "fused_merge": bool(b.plan["fused_combine"]) and args.path == "step",
                   "bytes_per_step": step_bytes,
                   "cold_cache_flush": m["flush"]},
        "roofline": {"bound": "hbm", "kernel": kernel_tag, "achieved": round(attn_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(attn_avg_ms * 1e3, 3),
                     "avg_launch_us_events": round(float(np.mean(attn_ms)) * 1e3, 3),
                     "launch_us_p10_p50_p90": [round(float(np.percentile(attn_ms, q)) * 1e3, 2) for q in (10, 50, 90)],
                     "bytes_per_launch": attn_bytes,
                     "traffic": traffic},
        "cpu_baseline": None,
    }
    ku = m["kernel_us"]
    if ku and ku.get("attn_split"):
        rec["roofline"]["kernel_us_profiler"] = round(float(np.mean(ku["attn_split"])), 3)

    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a sample", file=sys.stderr, flush=True)

        def host_layer_fn(l):
            L = b.layers[l]

            def u16(t):
                return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            return (u16(L["q"]), u16(L["k_cache"]), u16(L["v_cache"]), u16(L["k_new"]),
                    u16(L["v_new"]), L["seq_pos"].cpu().numpy(),
                    u16(L["out_gate"]) if "out_gate" in L else None)
        rec["cpu_baseline"] = cpu_baseline(w, host_layer_fn, w.layers, args.cpu_seconds,
                                           None if b.freqs is None else b.freqs.cpu().numpy(),
                                           None if b.block_table is None else b.block_table.cpu().numpy())

    if configs == "all":
        # Every other workload runs in a child process of its own, as it would run
        # alone: measured after the default workload's 30 GB in this process, the same kernels
        # took 4-5% longer (where the caching allocator then places a workload's
        # caches changes its streaming rate).
        del b
        torch.cuda.empty_cache()
        rec["configs"] = {}
        for name, wc in WORKLOADS.items():
            if name == w.name:
                continue
            print(f"[bench] config {name}", file=sys.stderr, flush=True)
            cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--config-record",
                   "--steps", str(args.config_steps), "--warmup", str(args.warmup)]
            if args.no_kernel_profiler:
                cmd.append("--no-kernel-profiler")
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
            lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
            if r.returncode != 0 or not lines:
                sys.stderr.write(r.stderr[-2000:])
                raise SystemExit(f"bench.py: workload {name} failed (exit {r.returncode})")
            rec["configs"][name] = json.loads(lines[-1])

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
