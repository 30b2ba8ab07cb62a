#!/usr/bin/env python3
"""Benchmark of the top-k selection / top-K sparse-attention decode hot path
on one MI355X.

Headline ("value", one "step"): one top-K sparse-attention decode step of
the mha-32k workload -- B16 H32 D128, context 32768, bf16 q, K, V ~ N(0, 1)
with 64 planted keys per head, scores q K^T / sqrt(128) in fp32, Top-512 via
(b, k_b) = (256, 2), softmax-V over the selected keys -- the largest of the
workloads (4.36 GB of algorithmic bytes per step).  value = scores per second
(B * H * L / step time); ms_per_step is the decode time of one step.

The same run measures every other workload of the path the same way and
reports each under "workloads": vocab-128k (256 x 131072 bf16, k = 64:
exact, (64, 1), (128, 2) + final), gqa-128k (B4 Hq32 Hkv8, context 131072,
Top-512 via (512, 4) + final, exact and rerank), wide-1m (64 x 2^20 fp32,
k = 8192: exact and (512, 16) + final) and sel-4k (1 x 4096 fp32, k = 64).

Timing: K calls per mode back to back on torch's stream (the library's
stream), queued behind a spin kernel so that the GPU never waits for the
host, bracketed by HIP events on that stream; selection inputs rotate over
enough copies (640 MB) that no call finds its input in the 256 MB Infinity
Cache (decode caches are larger than it).  Per-kernel times (the stages of a
call: scoring + stage 1, stage 2 + softmax-V, ...) come from HIP events the
library records after each of its kernels (atopk_stage_events) in a second
pass of the same calls.  "roofline" gives, per workload, the dominant
kernel's algorithmic bytes per launch over its event-timed launch duration
against the 8 TB/s HBM peak, and the HBM traffic rocprofv3 counted for it
(profiles/traffic_*.md) while its sources are unchanged.  The CPU oracle
(numpy, float64 for the decode) runs on a bounded sample of every workload
in a process pool over the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only MODE]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "top-k score elements/s + HBM GB/s vs peak; recall vs Eq.(1); decode µs/step"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
CSRC = os.path.join(ROOT, "top_sparse_attention_exact_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    help="all | core (the five workloads, no secondary legs) | mha | gqa | vocab | wide | sel4k | "
                         "assign | tradeoff | graph | stream | sweep (not in all) | copy")
    ap.add_argument("--no-flush", action="store_true", help="no cache flush before the single-call latency runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-kernel (stage) timing pass")
    ap.add_argument("--cpu-seconds", type=float, default=5.0, help="CPU oracle budget per workload (wall seconds)")
    return ap.parse_args()


# ------------------------------------------------------------ traffic ----

def source_hash(sources):
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(name):
    """(kernel, HBM bytes per launch) from the committed rocprofv3 counter
    summary profiles/traffic_<name>.md, if the sources it lists still hash
    the same (None once the kernel changed since the counters were taken)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.md" % name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            key, val = line.strip()[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    sources = [s.strip() for s in fields.get("kernel_sources", "").split(",") if s.strip()]
    if not sources or fields.get("kernel_source_hash") != source_hash(sources):
        return None
    try:
        return fields.get("kernel"), int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class EventTimer:
    """Times library calls with HIP events on torch's current stream (the
    stream the library launches on).

    stream(): K launches per call back to back, queued behind a spin kernel
    long enough that the whole batch is queued before the GPU reaches it
    (checked: the first event must still be pending when queueing ends; the
    spin grows and the batch is re-run otherwise).  Gives the average launch
    duration with no host gaps.

    cold(): one call at a time after a cache flush.  The flush READS 1 GiB
    (more than the 4 MB-per-XCD L2 plus the 256 MB Infinity Cache), leaving
    only clean lines: a write-based flush leaves dirty lines whose
    write-back would compete with the timed reads."""

    def __init__(self, flush):
        import torch

        self.torch = torch
        self.flush = flush
        self.flush_buf = None
        self.spin = 1 << 21

    def stream(self, calls, steps, warmup):
        torch = self.torch
        for w in range(warmup):
            for _, fn in calls:
                fn(w)
        torch.cuda.synchronize()
        for _ in range(5):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            torch.cuda._sleep(self.spin)
            first = torch.cuda.Event(enable_timing=True)
            first.record()
            ev = {}
            for name, fn in calls:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for s in range(steps):
                    fn(s)
                e1.record()
                ev[name] = (e0, e1)
            ahead = not first.query()
            last = ev[calls[-1][0]][1]
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            if ahead:
                break
            self.spin *= 4
        us = {name: e0.elapsed_time(e1) * 1e3 / steps for name, (e0, e1) in ev.items()}
        gpu_s = first.elapsed_time(last) * 1e-3
        return us, {"gpu_s": gpu_s, "wall_s": wall, "queued_ahead": ahead}

    def cold(self, calls, steps, warmup):
        torch = self.torch
        if self.flush and self.flush_buf is None:
            self.flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        for w in range(warmup):
            for _, fn in calls:
                fn(w)
        torch.cuda.synchronize()
        pairs = {name: [] for name, _ in calls}
        for s in range(steps):
            for name, fn in calls:
                if self.flush_buf is not None:
                    self.flush_sink = self.flush_buf.sum()
                torch.cuda._sleep(20000)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn(s)
                e1.record()
                pairs[name].append((e0, e1))
        torch.cuda.synchronize()
        return {name: [a.elapsed_time(b) * 1e3 for a, b in v] for name, v in pairs.items()}


def copies(x, min_bytes):
    """x plus clones of it, together at least min_bytes."""
    nb = x.numel() * x.element_size()
    r = max(1, -(-min_bytes // nb))
    return [x] + [x.clone() for _ in range(r - 1)]


ROTATE_BYTES = 640 << 20


def stage_split(fn, steps, spin):
    """Per-kernel durations of a library call: the caller records an event
    before the call and the library records one after each of its kernels
    (atopk_stage_events), all on torch's current stream, the calls queued
    behind a spin kernel.  Returns (mean µs per kernel, per-call lists)."""
    import numpy as np
    import torch

    import top_sparse_attention_exact_amd as atk

    probe = [torch.cuda.Event(enable_timing=True) for _ in range(64)]
    for e in probe:
        e.record()
    torch.cuda.synchronize()
    atk.stage_events(probe)
    fn(0)
    nk = min(atk.stage_count(), len(probe))
    atk.stage_events(None)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    torch.cuda._sleep(spin)
    for s in range(steps):
        evs[s][0].record()
        atk.stage_events(evs[s][1:])
        fn(s)
    atk.stage_events(None)
    torch.cuda.synchronize()
    per = [[evs[s][j].elapsed_time(evs[s][j + 1]) * 1e3 for j in range(nk)] for s in range(steps)]
    return [float(np.mean([p[j] for p in per])) for j in range(nk)], per


def describe_stages(names, alg, us):
    """Stage list of one call: kernel names (when the call launched the
    expected number of kernels), algorithmic bytes and event-timed µs."""
    if len(names) != len(us):
        names = ["kernel %d" % j for j in range(len(us))]
        alg = [None] * len(us)
    out = []
    for nm, a, t in zip(names, alg, us):
        d = {"kernel": nm, "us": round(t, 2)}
        if a is not None:
            d["alg_bytes"] = a
            d["gbps"] = a / (t * 1e-6) / 1e9
            d["frac_hbm_peak"] = d["gbps"] / HBM_PEAK_GBPS
        out.append(d)
    return out


def roofline_block(stages, call_alg, call_us, traffic_name):
    """Roofline of one call: its dominant kernel (the one with the largest
    share of the call's kernel time) when that kernel carries algorithmic
    bytes of its own and at least 75% of the time, else the whole call."""
    if len(stages) == 1:
        # one kernel per call: the back-to-back stream time of the calls is
        # that kernel's average launch duration (the stage pass adds an event
        # record between launches)
        stages = [dict(stages[0], us=call_us)]
    total = sum(s["us"] for s in stages) if stages else call_us
    dom = max(stages, key=lambda s: s["us"]) if stages else None
    if dom is not None and "alg_bytes" in dom and dom["us"] >= 0.75 * total:
        kernel, alg, us = dom["kernel"], dom["alg_bytes"], dom["us"]
    else:
        # the whole call, timed back to back (the stage events add their own
        # overhead between the kernels)
        kernel = " + ".join(s["kernel"] for s in stages) if stages else "whole call"
        alg, us = call_alg, call_us
    achieved = alg / (us * 1e-6) / 1e9
    rec = recorded_traffic(traffic_name)
    traffic = rec[1] if rec is not None and rec[0] == kernel else None
    return {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "alg_bytes_per_launch": alg, "launch_us": round(us, 2), "call_us": round(call_us, 2)}


def cold_stats(vals):
    import numpy as np

    return {"us_cold_median": round(float(np.median(vals)), 2), "us_cold_p10": round(float(np.percentile(vals, 10)), 2),
            "us_cold_p90": round(float(np.percentile(vals, 90)), 2)}


# Kernels each call launches, in order, with the algorithmic bytes each one
# carries: the input read goes to the kernel that reads it first, the output
# write to the kernel that writes it; work the path adds on top of the
# definition (a re-read, lists in the workspace) carries none.
def selection_kernels(workload, mode, m, n, k, es, width):
    read, write = m * n * es, m * width * (es + 4)
    if workload == "vocab-128k":
        name = {"exact": "row_exact_kernel<1>", "b64k1": "row_bucket_bf16_kernel<1, false>",
                "b128k2_final": "row_bucket_bf16_kernel<2, true>"}[mode]
        return [name], [read + write]
    if workload == "wide-1m":
        if mode == "exact":
            return (["wide_sample_kernel", "wide_collect_row_kernel", "wide_final_kernel"], [0, read, write])
        return (["wide_onepass_kernel", "wide_final_kernel"], [read, write])
    return [], []


def decode_kernels(c, mode, group, nkernels=2):
    """Scoring + stage 1, then the finish.  Both workloads plan at most one
    (head, bucket) pair per thread (the scoring kernel's first template
    argument); the exact Top-K runs the certified plan with k_b = 8.  One
    kernel: the scoring workgroups finished their heads in place (b k_b = K,
    one workgroup per head), so that kernel carries the V gather and the
    output too."""
    kbytes = c["bsz"] * c["hkv"] * c["ctx"] * c["d"] * 2
    qbytes = c["bsz"] * c["hq"] * c["d"] * 2
    vbytes = c["bsz"] * c["hq"] * c["k_sel"] * c["d"] * 2
    score = "decode_select_mfma_kernel<1, %d>" if group > 1 else "decode_select_kernel<1, %d>"
    kb = c["kb"] if mode == "bucketed" else 8
    if nkernels == 1:
        return [score % kb], [kbytes + 2 * qbytes + vbytes]
    nb = c["b"] if mode == "bucketed" else 256  # the certified plan's b on both decode workloads
    mp = 4 if nb * kb <= 2048 else 16  # the finish's compaction slots per thread
    return [score % kb, "decode_finish_kernel<%d, %d>" % (kb, mp)], [kbytes + qbytes, vbytes + qbytes]


def run_selection(args, timer, name):
    """One selection workload: every mode timed back to back over rotating
    copies, single-call latency after a cache flush, per-kernel stages."""
    import numpy as np
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    c = workloads.SELECTION[name]
    m, n, k = c["m"], c["n"], c["k"]
    if name == "vocab-128k":
        x = workloads.rows_normal_bf16(m, n, 2.0, seed=0, device="cuda")
    elif name == "wide-1m":
        x = workloads.rows_planted_residues(m, n, 512, k, seed=0, device="cuda")
    else:
        x = workloads.rows_uniform(m, n, seed=0, device="cuda")
    es = x.element_size()
    xs = copies(x, ROTATE_BYTES)
    torch.cuda.synchronize()
    outs = {}

    def mk(mode, f):
        def call(i):
            outs[mode] = f(xs[i % len(xs)])
        return mode, call

    calls = [mk("exact", lambda t: atk.exact(t, k))]
    widths = {"exact": k}
    for b, kb, fin in c["modes"]:
        mode = "b%dk%d%s" % (b, kb, "_final" if fin else "")
        calls.append(mk(mode, lambda t, b=b, kb=kb, fin=fin: atk.bucketed(t, k, b, kb, fin)))
        widths[mode] = k if fin else b * kb
    steps = args.steps if name == "vocab-128k" else max(3, min(args.steps, 10))
    us, info = timer.stream(calls, steps, args.warmup)
    cold = timer.cold(calls, max(3, min(args.steps, 10)), 1)
    res = {"m": m, "n": n, "k": k, "dtype": "bf16" if es == 2 else "f32", "input_copies": len(xs),
           "queued_ahead": info["queued_ahead"], "modes": {}}
    for mode, fn in calls:
        t = us[mode] * 1e-6
        alg = m * n * es + m * widths[mode] * (es + 4)
        d = {"us": round(us[mode], 2), "elements_per_s": m * n / t, "rows_per_s": m / t, "alg_bytes": alg,
             "gbps": alg / t / 1e9, "frac_hbm_peak": alg / t / 1e9 / HBM_PEAK_GBPS,
             "us_cold": round(float(np.mean(cold[mode])), 2), **cold_stats(cold[mode])}
        if not args.no_stages and name != "sel-4k":
            st_us, _ = stage_split(fn, max(3, min(args.steps, 10)), timer.spin)
            names, algs = selection_kernels(name, mode, m, n, k, es, widths[mode])
            d["stages"] = describe_stages(names, algs, st_us)
        res["modes"][mode] = d
    # recall of the bucketed modes against the exact result (index recall and,
    # for ties at the k-th value, value recall), with the recall models
    if "exact" in outs:
        import oracle

        ev, ei = outs["exact"]
        ex = ei.cpu().numpy()
        exv = ev.float().cpu().numpy().astype(np.float64)
        rec = {}
        for b, kb, fin in c["modes"]:
            mode = "b%dk%d%s" % (b, kb, "_final" if fin else "")
            bv, bi = outs[mode]
            got = bi.cpu().numpy()
            r = {"index_recall": float(np.mean([len(np.intersect1d(a, e)) / k for a, e in zip(got, ex)])),
                 "value_recall": float(oracle.value_recall(bv.float().cpu().numpy().astype(np.float64), exv).mean()),
                 "eq1": oracle.eq1(k, b, kb), "eq1_finite_n": oracle.eq1_finite(n, k, b, kb)}
            if name == "wide-1m":
                rr = oracle.recall(got, ex)
                r["index_recall_iid_rows"] = float(rr[0::2].mean())
                r["index_recall_adversarial_rows"] = float(rr[1::2].mean())
                r["eq2_worst_case"] = oracle.eq2(n, k, b, kb)
            rec[mode] = r
        res["recall"] = rec
    res["_x"] = x
    del xs
    return res


def run_decode(args, timer, name):
    """One decode workload: bucketed and exact Top-K (and, on gqa-128k, the
    candidate rerank) timed back to back, per-kernel stages."""
    import numpy as np
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    c = workloads.DECODE[name]
    if name == "mha-32k":
        q, K, V, _ = workloads.decode_mha(c["bsz"], c["hq"], c["ctx"], c["d"], 64, 0.8, seed=0, device="cuda")
    else:
        q, K, V, _ = workloads.decode_gqa(c["bsz"], c["hq"], c["hkv"], c["ctx"], c["d"], 0.01, 3.0, seed=0,
                                          device="cuda")
    torch.cuda.synchronize()
    group = c["hq"] // c["hkv"]
    modes = [("bucketed", c["b"], c["kb"]), ("exact", 1, c["k_sel"])]
    calls = [(mode, (lambda i, b=b, kb=kb: atk.sparse_attn_decode(q, K, V, c["k_sel"], b, kb)))
             for mode, b, kb in modes]
    cand = None
    if name == "gqa-128k":
        # Candidate rerank on the same cache: per query head 4 retrieved
        # supports of K_sel positions (seeded uniform draws, repeats allowed)
        # united with the last K_sel keys, exact Top-K_sel inside.
        g = torch.Generator(device="cpu").manual_seed(11)
        ncand = RERANK_SUPPORTS * c["k_sel"]
        cand = torch.randint(0, c["ctx"], (c["bsz"], c["hq"], ncand), generator=g, dtype=torch.int32).cuda()
        calls.append(("rerank", lambda i: atk.sparse_attn_rerank(q, K, V, cand, c["k_sel"], c["k_sel"])))
    steps = max(3, min(args.steps, 10))
    us, info = timer.stream(calls, steps, 2)
    kbytes = K.numel() * 2
    alg = kbytes + q.numel() * 2 + c["bsz"] * c["hq"] * c["k_sel"] * c["d"] * 2 + q.numel() * 2
    res = {"B": c["bsz"], "Hq": c["hq"], "Hkv": c["hkv"], "L": c["ctx"], "D": c["d"], "K_sel": c["k_sel"],
           "b": c["b"], "kb": c["kb"], "alg_bytes": alg, "queued_ahead": info["queued_ahead"], "modes": {}}
    for mode, fn in calls:
        if mode == "rerank":
            continue
        t = us[mode] * 1e-6
        d = {"us_per_step": round(us[mode], 1), "gbps": alg / t / 1e9, "frac_hbm_peak": alg / t / 1e9 / HBM_PEAK_GBPS,
             "scores_per_s": c["bsz"] * c["hq"] * c["ctx"] / t}
        if not args.no_stages:
            st_us, _ = stage_split(fn, steps, timer.spin)
            names, algs = decode_kernels(c, mode, group, len(st_us))
            d["stages"] = describe_stages(names, algs, st_us)
        res["modes"][mode] = d
    if cand is not None:
        heads = c["bsz"] * c["hq"]
        nuniq = sum(len(np.union1d(row, np.arange(c["ctx"] - c["k_sel"], c["ctx"])))
                    for row in cand.view(heads, -1).cpu().numpy())
        ralg = nuniq * c["d"] * 2 + heads * (c["k_sel"] * c["d"] * 2 + cand.shape[2] * 4 + 2 * c["d"] * 2)
        t = us["rerank"] * 1e-6
        res["modes"]["rerank"] = {"us_per_step": round(us["rerank"], 1), "supports": RERANK_SUPPORTS,
                                  "window": c["k_sel"], "mean_candidates": nuniq / heads, "alg_bytes": ralg,
                                  "gbps": ralg / t / 1e9, "frac_hbm_peak": ralg / t / 1e9 / HBM_PEAK_GBPS,
                                  "speedup_vs_exact": us["exact"] / us["rerank"]}
    res["_qkv"] = (q, K, V)
    return res


RERANK_SUPPORTS = 4


# ------------------------------------------------------ CPU oracle leg ----
# Run in a process pool created before the GPU is touched ("spawn": fresh
# interpreters that import numpy and the oracle only).

def cpu_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or platform.machine()


def _cpu_selection_task(task):
    """Oracle on one block of rows, every mode of the workload."""
    import oracle

    rows, tag, k, modes = task
    oracle.exact_topk(rows, k, tag)
    for b, kb, fin in modes:
        oracle.bucketed_topk(rows, k, b, kb, fin, tag)
    return rows.shape[0] * rows.shape[1] * (1 + len(modes))


def _cpu_decode_task(task):
    """float64 dense-then-masked decode of the query heads that share one KV
    head, in the workload's (b, k_b) mode."""
    import oracle

    q_bits, k_bits, v_bits, scale, k_sel, b, kb = task
    oracle.attn_decode(q_bits[None], k_bits[None, None], v_bits[None, None], scale, k_sel, b, kb)
    return q_bits.shape[0] * k_bits.shape[0]


def cpu_run(pool, cores, fn, tasks, seconds):
    """Tasks in waves of `cores` until the time budget is spent (at least one
    wave).  Returns (units per second, tasks done, wall seconds)."""
    t0 = time.perf_counter()
    done = units = 0
    while done < len(tasks) and (done == 0 or time.perf_counter() - t0 < seconds):
        wave = tasks[done:done + cores]
        units += sum(pool.map(fn, wave))
        done += len(wave)
    dt = time.perf_counter() - t0
    return units / dt, done, dt


def cpu_leg(pool, cores, sel, dec, seconds):
    """The CPU oracle (as it stands) on the same bytes as the GPU runs, per
    workload, over `cores` worker processes."""
    import numpy as np
    import torch

    from top_sparse_attention_exact_amd import workloads

    out = {}
    for name, r in sel.items():
        c = workloads.SELECTION[name]
        x = r["_x"]
        per = 1 if c["n"] >= 1 << 20 else (4 if c["n"] >= 1 << 16 else 64)
        rows = min(c["m"], per * cores * 8)
        if x.dtype == torch.bfloat16:
            hx, tag = x[:rows].cpu().view(torch.int16).numpy().view(np.uint16), "bf16"
        else:
            hx, tag = x[:rows].cpu().numpy(), "f32"
        if name == "sel-4k":  # one row at the workload's size: more seeded rows of the same recipe
            hx = workloads.rows_uniform(per * cores * 4, c["n"], seed=1, device="cpu").numpy()
        tasks = [(hx[i:i + per], tag, c["k"], c["modes"]) for i in range(0, hx.shape[0], per)]
        rate, done, dt = cpu_run(pool, cores, _cpu_selection_task, tasks, seconds)
        out[name] = {"value": rate, "unit": "elements/s", "cores": cores, "kind": "oracle",
                     "sample": "%d rows x %d, exact + %d bucketed modes per row, %.1f s wall" % (
                         min(done * per, hx.shape[0]), c["n"], len(c["modes"]), dt)}
    for name, r in dec.items():
        c = workloads.DECODE[name]
        q, K, V = r["_qkv"]
        g = c["hq"] // c["hkv"]
        scale = float(np.float32(1.0 / math.sqrt(c["d"])))
        per_wave = cores
        groups = [(i, h) for i in range(c["bsz"]) for h in range(c["hkv"])][:per_wave * 4]
        b16 = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
        tasks = [(b16(q[i, h * g:(h + 1) * g]), b16(K[i, h]), b16(V[i, h]), scale, c["k_sel"], c["b"], c["kb"])
                 for i, h in groups]
        rate, done, dt = cpu_run(pool, cores, _cpu_decode_task, tasks, seconds)
        out[name] = {"value": rate, "unit": "scores/s", "cores": cores, "kind": "oracle",
                     "sample": "%d of %d query heads (float64 dense-then-masked decode, (b, k_b) = (%d, %d)), "
                               "%.1f s wall" % (done * g, c["bsz"] * c["hq"], c["b"], c["kb"], dt)}
    return out


def assignment_compare(args, timer):
    """Runtime of contiguous against interleaved buckets on the vocab-128k
    batch (the comparison of Figure 8 on the Approximate Top-k page), and
    their recall on AR(1) rows of correlation 0.99 (Figure 6)."""
    import numpy as np
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    cfg = workloads.SELECTION["vocab-128k"]
    m, n, k = cfg["m"], cfg["n"], cfg["k"]
    x = workloads.rows_normal_bf16(m, n, 2.0, seed=0, device="cuda")
    xs = copies(x, ROTATE_BYTES)
    calls = []
    for b, kb, fin in cfg["modes"]:
        for assign in ("interleaved", "contiguous"):
            calls.append(("b%dk%d%s_%s" % (b, kb, "_final" if fin else "", assign),
                          (lambda i, b=b, kb=kb, fin=fin, a=assign: atk.bucketed(xs[i % len(xs)], k, b, kb, fin,
                                                                                  assignment=a))))
    torch.cuda.synchronize()
    us, info = timer.stream(calls, max(3, min(args.steps, 20)), 2)
    out = {"workload": "vocab-128k", "queued_ahead": info["queued_ahead"]}
    for name, _ in calls:
        out[name] = {"us": round(us[name], 2), "frac_hbm_peak": (m * n * 2) / (us[name] * 1e-6) / 1e9 / HBM_PEAK_GBPS}
    del x, xs
    ar = workloads.rows_ar1(64, n, 0.99, seed=0, device="cuda")
    _, ex = atk.exact(ar, k)
    ex = ex.cpu().numpy()
    rec = {}
    for assign in ("interleaved", "contiguous"):
        _, idx = atk.bucketed(ar, k, 64, 1, False, assignment=assign)
        got = idx.cpu().numpy()
        rec[assign] = float(np.mean([len(np.intersect1d(a, e)) / k for a, e in zip(got, ex)]))
    out["recall_ar1_rho0.99_b64k1"] = rec
    torch.cuda.empty_cache()
    return out


def tradeoff(args, timer):
    """Runtime against recall of the bucketed top-k at the vocabulary-sampling
    and knowledge-graph shapes (Figure 4 of the Approximate Top-k page): the
    exact top-k, then every (b, k_b) of the sweep with the final exact top-k."""
    import numpy as np
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    res = {}
    for name, c in workloads.TRADEOFF.items():
        m, n, k = c["m"], c["n"], c["k"]
        x = workloads.rows_normal(m, n, c["std"], seed=0, device="cuda", workload=name)
        xs = copies(x, ROTATE_BYTES)
        torch.cuda.synchronize()
        _, ex = atk.exact(x, k)
        ex = ex.cpu().numpy()
        modes = workloads.tradeoff_modes(k)
        calls = [("exact", lambda i: atk.exact(xs[i % len(xs)], k))]
        for b, kb in modes:
            calls.append(("b%dk%d" % (b, kb), (lambda i, b=b, kb=kb: atk.bucketed(xs[i % len(xs)], k, b, kb, True))))
        us, info = timer.stream(calls, max(3, min(args.steps, 10)), 2)
        alg = m * n * 4 + m * k * 8
        out = {"m": m, "n": n, "k": k, "dtype": "f32", "input_copies": len(xs), "queued_ahead": info["queued_ahead"],
               "exact": {"us": round(us["exact"], 2), "frac_hbm_peak": alg / (us["exact"] * 1e-6) / 1e9 / HBM_PEAK_GBPS}}
        for b, kb in modes:
            nm = "b%dk%d" % (b, kb)
            _, idx = atk.bucketed(x, k, b, kb, True)
            got = idx.cpu().numpy()
            rec = float(np.mean([len(np.intersect1d(a, e)) / k for a, e in zip(got, ex)]))
            out[nm] = {"us": round(us[nm], 2), "recall": rec,
                       "frac_hbm_peak": alg / (us[nm] * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        # The measured chooser at three recall targets (its own timing).
        out["chooser"] = {}
        for target in (0.9, 0.95, 0.99):
            ch = atk.choose(x, k, target)
            out["chooser"][str(target)] = {"b": ch["b"], "kb": ch["kb"], "expected_recall": ch["recall"],
                                          "us": round(ch["us"], 2)}
        res[name] = out
        del x, xs
        torch.cuda.empty_cache()
    return res


def sweep(args, timer):
    """Runtime against n and k at m = 1 and m = 256 (Figures 15-16 of the
    Approximate Top-k page): the exact top-k and a bucketed top-k with
    k_b = 1 and b the smallest power of two >= 2k (at most 8192), final
    exact; torch.topk on the same rows is timed beside them as context."""
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    cfg = workloads.SWEEP
    pts = []
    for m in cfg["ms"]:
        for ln in cfg["log2n"]:
            n = 1 << ln
            if m * n * 4 > cfg["max_bytes"]:
                continue
            x = workloads.rows_normal(m, n, 1.0, seed=ln, device="cuda", workload="sweep")
            xs = copies(x, min(ROTATE_BYTES, 8 * m * n * 4))
            torch.cuda.synchronize()
            for k in cfg["ks"]:
                b = 1
                while b < 2 * k:
                    b *= 2
                b = min(b, 8192)
                if k > n or b * 1 < k or b > n:
                    continue
                calls = [("exact", lambda i, k=k: atk.exact(xs[i % len(xs)], k)),
                         ("bucketed", lambda i, k=k, b=b: atk.bucketed(xs[i % len(xs)], k, b, 1, True)),
                         ("torch.topk", lambda i, k=k: torch.topk(xs[i % len(xs)], k, dim=1))]
                us, _ = timer.stream(calls, max(3, min(args.steps, 10)), 2)
                pts.append({"m": m, "n": n, "k": k, "b": b, "exact_us": round(us["exact"], 2),
                            "bucketed_us": round(us["bucketed"], 2), "torch_topk_us": round(us["torch.topk"], 2)})
            del x, xs
            torch.cuda.empty_cache()
    return pts


def graph_leg(args, timer):
    """The selection step captured in a HIP graph (Figure 9 of the Approximate
    Top-k page) against the same calls launched one by one: host-side wall
    time per step with no spin ahead (launch cost included), for the
    vocab-128k step and the 1 x 4096 selection."""
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    res = {}
    for name in ("vocab-128k", "sel-4k"):
        c = workloads.SELECTION[name]
        m, n, k = c["m"], c["n"], c["k"]
        if name == "vocab-128k":
            x = workloads.rows_normal_bf16(m, n, 2.0, seed=0, device="cuda")
        else:
            x = workloads.rows_uniform(m, n, seed=0, device="cuda")
        xs = copies(x, ROTATE_BYTES)

        def step(t):
            atk.exact(t, k)
            for b, kb, fin in c["modes"]:
                atk.bucketed(t, k, b, kb, fin)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for t in xs[:2]:
                step(t)
        torch.cuda.current_stream().wait_stream(s)
        graphs = []
        for t in xs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(t)
            graphs.append(g)
        torch.cuda.synchronize()
        steps = max(20, args.steps * 10)
        out = {"m": m, "n": n, "k": k, "modes": ["exact"] + ["b%dk%d%s" % (b, kb, "_final" if f else "")
                                                            for b, kb, f in c["modes"]]}
        for mode in ("eager", "graph"):
            for i in range(3):
                graphs[i % len(graphs)].replay() if mode == "graph" else step(xs[i % len(xs)])
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record()
            for i in range(steps):
                graphs[i % len(graphs)].replay() if mode == "graph" else step(xs[i % len(xs)])
            e1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            out[mode] = {"wall_us_per_step": wall / steps * 1e6, "gpu_us_per_step": e0.elapsed_time(e1) * 1e3 / steps}
        # GPU time of the step queued ahead of the GPU (no host gaps), both ways.
        us, _ = timer.stream([("eager", lambda i: step(xs[i % len(xs)])),
                              ("graph", lambda i: graphs[i % len(graphs)].replay())], max(3, min(args.steps, 10)), 2)
        out["eager"]["queued_us_per_step"] = us["eager"]
        out["graph"]["queued_us_per_step"] = us["graph"]
        res[name] = out
        del graphs, x, xs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


STREAM_SIZES = (("64MiB", 64 << 20), ("256MiB", 256 << 20), ("1GiB", 1 << 30), ("4GiB", 4 << 30))


def stream_calibration(args, timer):
    """A plain streaming-read kernel (calib/stream_read.hip) at the input
    sizes of the workloads, best over five grid sizes: the rate a kernel
    that only reads its input reaches on this GPU, the practical ceiling the
    kernels are compared with beside the 8 TB/s peak.  Buffers below 640 MB
    rotate over copies (no launch finds its input in the Infinity Cache)."""
    import ctypes

    import torch

    from top_sparse_attention_exact_amd import build as _build

    calib = ctypes.CDLL(_build.CALIB)
    calib.atopk_calib_stream_read.restype = ctypes.c_int
    calib.atopk_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                               ctypes.c_void_p]
    block_counts = (1024, 2048, 4096, 8192, 16384)
    sink = torch.empty(max(block_counts), dtype=torch.int32, device="cuda")
    res = {}
    for name, nbytes in STREAM_SIZES:
        x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        xs = copies(x, ROTATE_BYTES)

        def call(i, xs=xs, nbytes=nbytes, blocks=1024):
            st = calib.atopk_calib_stream_read(ctypes.c_void_p(xs[i % len(xs)].data_ptr()), nbytes, blocks,
                                               ctypes.c_void_p(sink.data_ptr()),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError("stream read launch failed: %d" % st)

        calls = [("b%d" % nb, (lambda i, nb=nb: call(i, blocks=nb))) for nb in block_counts]
        us, _ = timer.stream(calls, max(3, min(args.steps, 10)), 2)
        best = min(us, key=us.get)
        res[name] = {"bytes": nbytes, "us": round(us[best], 2), "workgroups": int(best[1:]),
                     "gbps": nbytes / (us[best] * 1e-6) / 1e9,
                     "frac_hbm_peak": nbytes / (us[best] * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                     "us_by_workgroups": {k[1:]: round(v, 2) for k, v in us.items()}}
        del x, xs
        torch.cuda.empty_cache()
    return res


def copy_calibration(args, timer):
    """A plain elementwise copy (negation) of 256 MiB, the yardstick that
    scales the rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    nbytes = 256 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    us, _ = timer.stream([("copy", lambda i: torch.neg(src, out=dst))], max(3, min(args.steps, 10)), 1)
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": round(us["copy"], 2),
            "gbps": 2 * nbytes / us["copy"] / 1e3}


TRAFFIC_NAME = {("vocab-128k", "exact"): "vocab128k_exact", ("vocab-128k", "b64k1"): "vocab128k_b64k1",
                ("vocab-128k", "b128k2_final"): "vocab128k_b128k2", ("wide-1m", "b512k16_final"): "wide1m_b512k16",
                ("mha-32k", "bucketed"): "mha32k_bucketed", ("gqa-128k", "bucketed"): "gqa128k_bucketed"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (rows and heads shard with no "
              "communication across GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    only = args.only
    core = only in ("all", "core")
    want = {w: core or only == key for w, key in (("mha-32k", "mha"), ("gqa-128k", "gqa"), ("vocab-128k", "vocab"),
                                                  ("wide-1m", "wide"), ("sel-4k", "sel4k"))}
    pool = cores = None
    if not args.no_cpu_baseline and any(want.values()):
        import multiprocessing

        cores = cpu_cores()
        pool = multiprocessing.get_context("spawn").Pool(cores)  # before the GPU is touched
    import torch

    torch.cuda.set_device(0)
    timer = EventTimer(flush=not args.no_flush)
    if only == "copy":
        print(json.dumps({"copy_calibration": copy_calibration(args, timer)}), flush=True)
        return
    dec, sel = {}, {}
    for w in ("mha-32k", "gqa-128k"):
        if want[w]:
            dec[w] = run_decode(args, timer, w)
    for w in ("vocab-128k", "wide-1m", "sel-4k"):
        if want[w]:
            sel[w] = run_selection(args, timer, w)
    cpu = cpu_leg(pool, cores, sel, dec, args.cpu_seconds) if pool is not None else {}
    if pool is not None:
        pool.close()
        pool.join()
    for r in list(dec.values()) + list(sel.values()):
        r.pop("_x", None)
        r.pop("_qkv", None)
    torch.cuda.empty_cache()
    assign = assignment_compare(args, timer) if only in ("all", "assign") else None
    trade = tradeoff(args, timer) if only in ("all", "tradeoff") else None
    swp = sweep(args, timer) if only == "sweep" else None
    graph = graph_leg(args, timer) if only in ("all", "graph") else None
    stream = stream_calibration(args, timer) if only in ("all", "stream") else None

    # roofline per workload: the mode the workload names (bucketed decode,
    # the slowest vocab-128k mode, (512, 16) + final on wide-1m)
    roofs = {}
    for w, r in dec.items():
        d = r["modes"]["bucketed"]
        roofs[w] = roofline_block(d.get("stages", []), r["alg_bytes"], d["us_per_step"], TRAFFIC_NAME[(w, "bucketed")])
        roofs[w]["mode"] = "bucketed (%d, %d)%s" % (r["b"], r["kb"], " + final" if r["b"] * r["kb"] > r["K_sel"] else "")
    for w, r in sel.items():
        if w == "sel-4k":
            continue
        modes = r["modes"]
        mode = max(modes, key=lambda nm: modes[nm]["us"]) if w == "vocab-128k" else "b512k16_final"
        d = modes[mode]
        roofs[w] = roofline_block(d.get("stages", []), d["alg_bytes"], d["us"], TRAFFIC_NAME[(w, mode)])
        roofs[w]["mode"] = mode
    if stream is not None:
        sizes = {"vocab-128k": "64MiB", "wide-1m": "256MiB", "gqa-128k": "1GiB", "mha-32k": "4GiB"}
        for w, rf in roofs.items():
            rf["stream_read_gbps_same_size"] = stream[sizes[w]]["gbps"]

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if "mha-32k" in dec:
        r = dec["mha-32k"]
        d = r["modes"]["bucketed"]
        line.update({
            "value": d["scores_per_s"], "unit": "scores/s", "ms_per_step": d["us_per_step"] / 1e3,
            "config": {"workload": "mha-32k: Top-K sparse-attention decode, B16 H32 D128, context 32768, bf16 q/K/V "
                                   "~ N(0,1) with 64 keys per head planted at cosine 0.8; fp32 scores q.K/sqrt(128); "
                                   "Top-512 via (b, k_b) = (256, 2); softmax-V over the selected keys; one step = one "
                                   "decode call over all 512 heads (value = B*H*L scores per second)",
                       "B": r["B"], "H": r["Hq"], "D": r["D"], "L": r["L"], "K_sel": r["K_sel"], "b": r["b"],
                       "kb": r["kb"], "alg_bytes_per_step": r["alg_bytes"]},
            "roofline": roofs["mha-32k"],
        })
    elif sel or dec:
        w, r = next(iter({**dec, **sel}.items()))
        if w in dec:
            d = r["modes"]["bucketed"]
            line.update({"value": d["scores_per_s"], "unit": "scores/s", "ms_per_step": d["us_per_step"] / 1e3})
        else:
            d = r["modes"]["exact"]
            line.update({"value": d["elements_per_s"], "unit": "elements/s", "ms_per_step": d["us"] / 1e3})
        line["config"] = {"workload": w}
        if w in roofs:
            line["roofline"] = roofs[w]
    else:
        line.update({"value": None, "unit": None, "ms_per_step": None, "config": {"workload": only}})
    if roofs:
        line["rooflines"] = roofs
    if dec or sel:
        line["workloads"] = {**dec, **sel}
    if cpu:
        head = "mha-32k" if "mha-32k" in cpu else next(iter(cpu))
        line["cpu_baseline"] = dict(cpu[head])
        line["cpu_baseline"]["cpu_model"] = cpu_model()
        line["cpu_baseline"]["by_workload"] = {w: {k: v for k, v in c.items() if k in ("value", "unit", "sample")}
                                               for w, c in cpu.items()}
    if assign is not None:
        line["assignment"] = assign
    if trade is not None:
        line["tradeoff"] = trade
    if swp is not None:
        line["sweep"] = swp
    if graph is not None:
        line["graph"] = graph
    if stream is not None:
        line["stream_read"] = stream
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
