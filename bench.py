#!/usr/bin/env python3
"""Benchmark of the top-k selection hot path on one MI355X.

Workload (one "step"): the 256 x 131072 bf16 vocabulary-sampling batch
(N(0, 2^2) logits, k = 64) through every selection mode of the path:
exact top-64, bucketed (b, k_b) = (64, 1) without the final stage, and
bucketed (128, 2) with the final exact top-64.  Inputs are resident in HBM
before timing starts.

Throughput ("value", "us" per mode): K launches per mode back to back on one
stream, queued behind a spin kernel so that the GPU never waits for the
host, bracketed by HIP events on that stream; the launches rotate over
enough copies of the batch (640 MB) that no launch finds its input in the
256 MB Infinity Cache.  Latency ("us_cold"): single calls with HIP events
around each, after a 1 GiB read that evicts the L2 and the Infinity Cache
(timing protocol after the benchmark protocol printed with "Approximate
Top-k for Increased Parallelism": warm-up, then events around each top-k
launch queued behind a short spin kernel).

The same run also times the sparse-attention decode steps (scoring, Top-K
selection, softmax-V) of the two decode workloads, the small-row and
wide-row selection workloads, and the CPU oracle on a bounded sample of the
selection batch.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only MODE]
"""

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "top-k score elements/s + HBM GB/s vs peak; recall vs Eq.(1); decode µs/step"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    help="all | sel | exact | b64k1 | b128k2 | decode | mha | gqa | sel4k | wide | assign | tradeoff | graph "
                         "| stream | sweep (not in all) | copy")
    ap.add_argument("--no-flush", action="store_true", help="no cache flush before the single-call latency runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    return ap.parse_args()


# Sources the selection kernels of the step are compiled from.
KERNEL_SOURCES = ("common.h", "select_row.hip")


def kernel_source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "top_sparse_attention_exact_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    the named kernel, if the kernel sources still hash the same."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.md" % name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            key, val = line.strip()[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
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


def selection_step(args, timer):
    import numpy as np
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    cfg = workloads.SELECTION["vocab-128k"]
    m, n, k = cfg["m"], cfg["n"], cfg["k"]
    x = workloads.rows_normal_bf16(m, n, 2.0, seed=0, device="cuda")
    xs = copies(x, ROTATE_BYTES)
    torch.cuda.synchronize()
    outs = {}

    def mk(name, f):
        def call(i):
            outs[name] = f(xs[i % len(xs)])
        return name, call

    calls = []
    if args.only in ("all", "sel", "exact"):
        calls.append(mk("exact", lambda t: atk.exact(t, k)))
    if args.only in ("all", "sel", "b64k1"):
        calls.append(mk("b64k1", lambda t: atk.bucketed(t, k, 64, 1, False)))
    if args.only in ("all", "sel", "b128k2"):
        calls.append(mk("b128k2", lambda t: atk.bucketed(t, k, 128, 2, True)))
    if not calls:
        return None
    us, info = timer.stream(calls, args.steps, args.warmup)
    cold = timer.cold(calls, max(3, min(args.steps, 10)), 1)
    width = {"exact": k, "b64k1": 64, "b128k2": k}
    modes = {}
    for name, _ in calls:
        t = us[name] * 1e-6
        alg = m * n * 2 + m * width[name] * (2 + 4)
        modes[name] = {
            "us": round(us[name], 2),
            "us_cold": round(float(np.mean(cold[name])), 2),
            "us_cold_median": round(float(np.median(cold[name])), 2),
            "us_cold_p10": round(float(np.percentile(cold[name], 10)), 2),
            "us_cold_p90": round(float(np.percentile(cold[name], 90)), 2),
            "elements_per_s": m * n / t,
            "alg_bytes": alg,
            "gbps": alg / t / 1e9,
            "frac_hbm_peak": alg / t / 1e9 / HBM_PEAK_GBPS,
        }
    recall = {}
    if "exact" in outs:
        ex = outs["exact"][1].cpu().numpy()
        for name in ("b64k1", "b128k2"):
            if name in outs:
                got = outs[name][1].cpu().numpy()
                r = [len(np.intersect1d(a, e)) / k for a, e in zip(got, ex)]
                recall[name] = float(np.mean(r))
    step_s = sum(modes[nm]["us"] for nm in modes) * 1e-6
    return dict(m=m, n=n, k=k, modes=modes, step_s=step_s, info=info, recall=recall, x=x, copies=len(xs))


RERANK_SUPPORTS = 4


def decode_steps(args, timer):
    import numpy as np
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    res = {}
    todo = [w for w in ("mha", "gqa") if args.only in ("all", "decode", w)]
    for w in todo:
        if w == "mha":
            c = workloads.DECODE["mha-32k"]
            q, K, V, _ = workloads.decode_mha(c["bsz"], c["hq"], c["ctx"], c["d"], 64, 0.8, seed=0, device="cuda")
        else:
            c = workloads.DECODE["gqa-128k"]
            q, K, V, _ = workloads.decode_gqa(c["bsz"], c["hq"], c["hkv"], c["ctx"], c["d"], 0.01, 3.0, seed=0,
                                              device="cuda")
        torch.cuda.synchronize()
        modes = [("bucketed", c["b"], c["kb"]), ("exact", 1, c["k_sel"])]
        calls = [(name, (lambda i, b=b, kb=kb: atk.sparse_attn_decode(q, K, V, c["k_sel"], b, kb)))
                 for name, b, kb in modes]
        if w == "gqa":
            # Candidate rerank on the same cache: per query head, 4 retrieved
            # supports of K_sel positions each (seeded uniform draws; repeats
            # allowed) united with the last K_sel keys, exact Top-K_sel inside.
            g = torch.Generator(device="cpu").manual_seed(11)
            ncand = RERANK_SUPPORTS * c["k_sel"]
            cand = torch.randint(0, c["ctx"], (c["bsz"], c["hq"], ncand), generator=g, dtype=torch.int32).cuda()
            calls.append(("rerank", lambda i: atk.sparse_attn_rerank(q, K, V, cand, c["k_sel"], c["k_sel"])))
        us, info = timer.stream(calls, max(3, min(args.steps, 10)), 2)
        kbytes = K.numel() * 2
        alg = kbytes + q.numel() * 2 + c["bsz"] * c["hq"] * c["k_sel"] * c["d"] * 2 + q.numel() * 2
        out = {"workload": "%s-%dk" % (w, c["ctx"] // 1024), "B": c["bsz"], "Hq": c["hq"], "Hkv": c["hkv"],
               "L": c["ctx"], "K_sel": c["k_sel"], "b": c["b"], "kb": c["kb"], "alg_bytes": alg,
               "queued_ahead": info["queued_ahead"]}
        for name, _, _ in modes:
            t = us[name] * 1e-6
            out[name] = {"us_per_step": round(us[name], 1), "gbps": alg / t / 1e9,
                         "frac_hbm_peak": alg / t / 1e9 / HBM_PEAK_GBPS,
                         "scores_per_s": c["bsz"] * c["hq"] * c["ctx"] / t}
        if w == "gqa":
            # Each head reads its unique candidates' K rows, its K_sel V rows
            # and its candidate list (plus q and out).
            heads = c["bsz"] * c["hq"]
            nuniq = sum(len(np.union1d(row, np.arange(c["ctx"] - c["k_sel"], c["ctx"])))
                        for row in cand.view(heads, -1).cpu().numpy())
            ralg = nuniq * c["d"] * 2 + heads * (c["k_sel"] * c["d"] * 2 + ncand * 4 + 2 * c["d"] * 2)
            t = us["rerank"] * 1e-6
            out["rerank"] = {"us_per_step": round(us["rerank"], 1), "supports": RERANK_SUPPORTS,
                             "window": c["k_sel"], "mean_candidates": nuniq / heads, "alg_bytes": ralg,
                             "gbps": ralg / t / 1e9, "frac_hbm_peak": ralg / t / 1e9 / HBM_PEAK_GBPS,
                             "speedup_vs_exact": us["exact"] / us["rerank"]}
        res[out["workload"]] = out
        del q, K, V
        torch.cuda.empty_cache()
    return res


def other_selection(args, timer):
    """The 1 x 4096 fp32 and 64 x 2^20 fp32 selection workloads (secondary)."""
    import torch

    import top_sparse_attention_exact_amd as atk
    from top_sparse_attention_exact_amd import workloads

    res = {}
    todo = [w for w in ("sel4k", "wide") if args.only in ("all", w)]
    for w in todo:
        if w == "sel4k":
            c = workloads.SELECTION["sel-4k"]
            x = workloads.rows_uniform(c["m"], c["n"], seed=0, device="cuda")
        else:
            c = workloads.SELECTION["wide-1m"]
            x = workloads.rows_planted_residues(c["m"], c["n"], 512, c["k"], seed=0, device="cuda")
        xs = copies(x, ROTATE_BYTES)
        m, n, k = c["m"], c["n"], c["k"]
        calls = [("exact", lambda i: atk.exact(xs[i % len(xs)], k))]
        for b, kb, fin in c["modes"]:
            calls.append(("b%dk%d%s" % (b, kb, "_final" if fin else ""),
                          (lambda i, b=b, kb=kb, fin=fin: atk.bucketed(xs[i % len(xs)], k, b, kb, fin))))
        torch.cuda.synchronize()
        us, info = timer.stream(calls, max(3, min(args.steps, 10)), 2)
        out = {"m": m, "n": n, "k": k, "dtype": "f32", "queued_ahead": info["queued_ahead"]}
        for name, _ in calls:
            t = us[name] * 1e-6
            alg = m * n * 4 + m * k * 8
            out[name] = {"us": round(us[name], 2), "elements_per_s": m * n / t, "gbps": alg / t / 1e9,
                         "frac_hbm_peak": alg / t / 1e9 / HBM_PEAK_GBPS}
        res["sel-4k" if w == "sel4k" else "wide-1m"] = out
        del x, xs
        torch.cuda.empty_cache()
    return res


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


def cpu_leg(sel, seconds):
    """The CPU oracle (as it stands) on a bounded sample of the same batch."""
    import numpy as np
    import torch

    import oracle

    x = sel["x"]
    m, n, k = sel["m"], sel["n"], sel["k"]
    hx = x.cpu().view(torch.int16).numpy().view(np.uint16)
    rows = 0
    t0 = time.perf_counter()
    while rows < m and (rows < 8 or time.perf_counter() - t0 < seconds):
        r = hx[rows:rows + 1]
        oracle.exact_topk(r, k, "bf16")
        oracle.bucketed_topk(r, k, 64, 1, False, "bf16")
        oracle.bucketed_topk(r, k, 128, 2, True, "bf16")
        rows += 1
    dt = time.perf_counter() - t0
    ref = {
        "b64k1": {"eq1": oracle.eq1(k, 64, 1), "eq1_finite_n": oracle.eq1_finite(n, k, 64, 1)},
        "b128k2": {"eq1": oracle.eq1(k, 128, 2), "eq1_finite_n": oracle.eq1_finite(n, k, 128, 2)},
    }
    return {
        "value": rows * n * 3 / dt,
        "unit": "elements/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d of %d rows of the step's batch, all three modes (numpy, one thread, %s)" % (
            rows, m, platform.processor() or platform.machine()),
    }, ref


# The kernel each selection mode of the step launches (one launch per call).
MODE_KERNEL = {"exact": "row_exact_kernel", "b64k1": "row_bucket_bf16_kernel<1, false>",
               "b128k2": "row_bucket_bf16_kernel<2, true>"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (rows and heads shard with no "
              "communication across GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    timer = EventTimer(flush=not args.no_flush)
    if args.only == "copy":
        print(json.dumps({"copy_calibration": copy_calibration(args, timer)}), flush=True)
        return
    sel = selection_step(args, timer) if args.only in ("all", "sel", "exact", "b64k1", "b128k2") else None
    dec = decode_steps(args, timer) if (not args.no_decode and args.only in ("all", "decode", "mha", "gqa")) else {}
    other = other_selection(args, timer) if args.only in ("all", "sel4k", "wide") else {}
    assign = assignment_compare(args, timer) if args.only in ("all", "assign") else None
    trade = tradeoff(args, timer) if args.only in ("all", "tradeoff") else None
    swp = sweep(args, timer) if args.only == "sweep" else None
    graph = graph_leg(args, timer) if args.only in ("all", "graph") else None
    stream = stream_calibration(args, timer) if args.only in ("all", "stream") else None

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if sel is not None:
        modes = sel["modes"]
        passes = len(modes)
        value = passes * sel["m"] * sel["n"] / sel["step_s"]
        dom = max(modes, key=lambda nm: modes[nm]["us"])
        line.update({
            "value": value,
            "unit": "elements/s",
            "ms_per_step": sel["step_s"] * 1e3,
            "config": {"workload": "vocab-128k: 256 x 131072 bf16 ~ N(0, 2^2), k = 64; one step = " +
                                   " + ".join(modes) + " (value counts m*n elements per mode)",
                       "m": sel["m"], "n": sel["n"], "k": sel["k"], "modes": list(modes),
                       "input_copies": sel["copies"]},
            "roofline": {"bound": "hbm", "kernel": MODE_KERNEL[dom] + " (" + dom + ")",
                         "achieved": modes[dom]["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": modes[dom]["gbps"] / HBM_PEAK_GBPS, "traffic": recorded_traffic(dom),
                         "alg_bytes_per_launch": modes[dom]["alg_bytes"], "launch_us": modes[dom]["us"]},
            "modes": modes,
            "recall": sel["recall"],
            "timing": {"gpu_ms_per_step": sel["info"]["gpu_s"] / args.steps * 1e3,
                       "wall_ms_per_step_incl_spin": sel["info"]["wall_s"] / args.steps * 1e3,
                       "queued_ahead": sel["info"]["queued_ahead"]},
        })
    elif not dec and not other:
        line.update({"value": None, "unit": "elements/s", "ms_per_step": None,
                     "config": {"workload": "vocab-128k" if assign or graph else
                                ("vocab-sampling, kg-2.65m" if trade else ("stream read" if stream else "sweep"))}})
    elif dec:
        first = next(iter(dec.values()))
        line.update({"value": first["bucketed"]["scores_per_s"], "unit": "scores/s",
                     "ms_per_step": first["bucketed"]["us_per_step"] / 1e3, "config": {"workload": first["workload"]}})
    else:
        name, first = next(iter(other.items()))
        line.update({"value": first["exact"]["elements_per_s"], "unit": "elements/s",
                     "ms_per_step": first["exact"]["us"] / 1e3, "config": {"workload": name}})
    if dec:
        line["decode"] = dec
    if other:
        line["other_selection"] = other
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
        if "roofline" in line:
            line["roofline"]["stream_read_64MiB_gbps"] = stream["64MiB"]["gbps"]
    if sel is not None and not args.no_cpu_baseline:
        cpu, ref = cpu_leg(sel, args.cpu_seconds)
        line["cpu_baseline"] = cpu
        for nm, r in ref.items():
            if nm in line["recall"]:
                line["recall"][nm] = {"measured": line["recall"][nm], **r}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
