#!/usr/bin/env python3
"""Benchmark of the block-quantized matvec / routed-MoE path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The default workload is the dense decode matvec the
metric is quoted on: Q8_0 and Q4_K weights, W 14336x4096 and 4096x14336, batches
of 1/2/4/8 tokens, activations quantized to Q8_1.  One step is one pass of the
whole path (activation quantize + quantized matvec) over all 16 cases.  Weights
are resident in HBM before timing; every case rotates over enough distinct
weight copies that no launch can be served from the 256 MB last-level cache.

The same line carries the rest of the metric under its own keys: routed-MoE layer
tokens/s for the Q4_K layer (1-4 tokens), the MXFP4 layer (1-512 tokens) and the
K-quant layer on the sorted tiles (512 tokens), and the grouped keep-quant GEMM
(512 tokens, Q5_K/Q6_K), each with its effective weight GB/s and HBM fraction.

Other workloads (--workload): q4_0_matvec, moe_q4k, moe_mxfp4, moe_kq_layer,
grouped_kq, and formats (every weight format x Q8_1 at W 14336x4096, 1/2/4/8
tokens; no CPU leg).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MOE_DTYPE = ("i8 x i8 -> i32 (v_dot4 on the Q4_K direct route, int8 MFMA on the K-quant tiles), "
             "E2M1 x FP8 halves of the i8 codes on the FP4 MFMA (MXFP4), f32 scale combine")
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 256 << 20         # calibration copy for the FETCH_SIZE / WRITE_SIZE counters


# sources the headline matvec kernel is compiled from
_HEADLINE_SRC = ("ft_mmvq.hip", "ft_mmvq_kernels.h", "ft_device.h", "ft_internal.h")


def _code_only(text):
    """C/C++ source without comments and blank lines (a comment edit does not change
    the kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def _src_hash():
    """Hash of the headline kernel's code (sources without comments): traffic figures
    are void once it changes."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_matvec_amd", "csrc")
    paths = [os.path.join(csrc, f) for f in _HEADLINE_SRC] + [os.path.join(ROOT, "include", "ft.h")]
    for path in paths:
        h.update(os.path.basename(path).encode())
        h.update(_code_only(open(path).read()).encode())
    return h.hexdigest()[:16]


def _traffic(key):
    """HBM bytes per launch measured with rocprofv3 counters (null if absent or stale)."""
    try:
        d = json.load(open(TRAFFIC_PATH))
    except (OSError, ValueError):
        return None
    e = d.get(key)
    if not e or e.get("src_hash") != _src_hash():
        return None
    return e["bytes_per_launch"]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_decode",
                    choices=["dense_decode", "q4_0_matvec", "moe_q4k", "moe_mxfp4", "moe_kq_layer", "grouped_kq",
                             "counters", "ceilings", "formats"])
    ap.add_argument("--dense-only", action="store_true",
                    help="dense_decode without the MoE and grouped-GEMM parts of the line")
    ap.add_argument("--copies", type=int, default=0, help="weight copies per matrix (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=str, default="", help="comma list overriding the token counts")
    ap.add_argument("--route", type=int, default=0, help="MoE route: 0 auto, 1 direct, 2 sorted tiles")
    ap.add_argument("--counters-scope", default="all", choices=["all", "headline"],
                    help="--workload counters: every kernel the counter summaries cover, or the headline only")
    ap.add_argument("--counters-summary", nargs="+", metavar="CSV",
                    help="per-kernel table of rocprofv3 --pmc CSVs of `--workload counters`")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of `--workload counters` into "
                         "profiles/traffic.json and exit")
    return ap.parse_args()


def main():
    args = _args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.counters_summary:
        counters_summary(args.counters_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "layout is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from block_quantized_matvec_amd import ft, synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    ft.lib()
    fn = {"dense_decode": bench_dense, "formats": bench_dense, "q4_0_matvec": bench_q4_0, "moe_q4k": bench_moe,
          "moe_mxfp4": bench_moe, "moe_kq_layer": bench_moe, "grouped_kq": bench_grouped, "counters": run_counters,
          "ceilings": lambda a, n, t, f, s: measure_ceilings(t, f)}[args.workload]
    out = fn(args, np, torch, ft, synth)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
_CAPTURE_STREAM = None


def _graph(torch, fn):
    """Capture fn() into a HIP graph on one dedicated stream.  fn runs once on that
    stream first, so the library's per-stream scratch pool is grown before capture."""
    global _CAPTURE_STREAM
    if _CAPTURE_STREAM is None:
        _CAPTURE_STREAM = torch.cuda.Stream()
    s = _CAPTURE_STREAM
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def measure_ceilings(torch, ft):
    """Ceilings measured on this part with the library's microkernels, best of 5 timed
    calls each: a streaming read of 4 GiB (GB/s), the int8 MFMA issue rate of the
    16x16x32 instruction the kernels use and of gfx950's 16x16x64 one, and the VALU
    dot4 rate (TOP/s), on 8 workgroups of 256 threads per CU."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        b = float("inf")
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            b = min(b, e0.elapsed_time(e1) / 1e3)
        return b

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    read = nbytes / best(lambda: ft.debug_ceiling("stream_read", buf, out=out)) / 1e9
    del buf
    waves = cus * 8 * 4
    im, idot = 4096, 16384
    mfma = waves * im * 8 * 16384 / best(lambda: ft.debug_ceiling("mfma_i8", iters=im, out=out)) / 1e12
    dot4 = waves * 64 * idot * 8 * 8 / best(lambda: ft.debug_ceiling("dot4", iters=idot, out=out)) / 1e12
    mfma64 = waves * im * 8 * 32768 / best(lambda: ft.debug_ceiling("mfma_i8_k64", iters=im, out=out)) / 1e12
    return {"stream_read_GBps": round(read, 1), "mfma_i8_TOPS": round(mfma, 1),
            "mfma_i8_k64_TOPS": round(mfma64, 1), "dot4_TOPS": round(dot4, 1), "stream_read_bytes": nbytes}


def _add_ceilings(out, torch, ft, tops=None):
    """Attach the measured ceilings and the roofline's fraction of the measured one
    (stream read for an HBM-bound line; tops: also the int8 MFMA fraction)."""
    ceil = measure_ceilings(torch, ft)
    out["ceilings"] = ceil
    rf = out["roofline"]
    rf["measured_peak"] = ceil["stream_read_GBps"]
    rf["frac_of_measured"] = round(rf["achieved"] / ceil["stream_read_GBps"], 4)
    if tops is not None:
        rf["mfma_frac_of_measured"] = round(tops / ceil["mfma_i8_TOPS"], 4)
    return out


def _time_graph(torch, g, reps):
    """Average replay time (s) of graph g, replayed `reps` times between two events."""
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def _time_graph_median(torch, g, reps=7):
    """Median over `reps` replays of graph g of one replay's time (s), each replay
    between its own two events on the launch stream (a host-side stall in one
    replay, e.g. a profiler flushing its buffers, does not enter the figure)."""
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(fn, sample_desc, unit, work, min_seconds=10.0, one_thread_seconds=4.0):
    """Time the oracle (as it stands) on the host cores: repeat fn until about
    min_seconds of CPU work with all the threads it has, report work per second;
    then the same on one thread for about one_thread_seconds."""
    import oracle

    def timed(limit):
        reps = 0
        t0 = time.perf_counter()
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= limit:
                return reps, dt

    threads = oracle.threads()
    reps, dt = timed(min_seconds)
    oracle.set_threads(1)
    try:
        reps1, dt1 = timed(one_thread_seconds)
    finally:
        oracle.set_threads(threads)
    return {"value": round(reps * work / dt, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {sample_desc}", "seconds": round(dt, 2), "cpu_model": _cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "one_thread": {"value": round(reps1 * work / dt1, 4), "sample": f"{reps1} x {sample_desc}",
                           "seconds": round(dt1, 2)}}


# ---------------------------------------------------------------------------
# dense decode matvec (the headline workload)
# ---------------------------------------------------------------------------
def bench_dense(args, np, torch, ft, synth):
    fmts_only = args.workload == "formats"
    cfg = synth.DECODE_FORMATS if fmts_only else synth.DENSE_DECODE
    tokens = [int(x) for x in args.tokens.split(",")] if args.tokens else list(cfg["tokens"])
    g = synth.rng(7, 1)
    mats = {}
    for fmt in cfg["formats"]:
        for (n, k) in cfg["shapes"]:
            W = synth.weights(fmt, n, k, g)
            mats[(fmt, n, k)] = W
    # every use of a matrix takes its next copy; a matrix has at least 8 copies and
    # enough that >= 600 MB of its other copies stream between two uses of one copy
    # (the last-level cache is 256 MB), also in the per-case graphs below, which
    # launch one case only
    total = sum(W.nbytes for W in mats.values())
    ncp = {key: args.copies or max(8, -(-600_000_000 // W.nbytes) + 1) for key, W in mats.items()}
    copies = max(ncp.values())
    dev = {key: [torch.from_numpy(W).cuda()] for key, W in mats.items()}
    for key in dev:
        base = dev[key][0]
        dev[key] += [base.clone() for _ in range(ncp[key] - 1)]
    # the activations of every token count at one K are the rows of one [sum t][K]
    # matrix, quantized by one launch per step; a case reads its rows
    ks = sorted({k for (_, _, k) in mats})
    row0 = {t: sum(tokens[:i]) for i, t in enumerate(tokens)}
    nrows = sum(tokens)
    xall = {k: synth.activations(nrows, k, g) for k in ks}
    dxall = {k: torch.from_numpy(v).cuda() for k, v in xall.items()}
    xqall = {k: torch.empty((nrows, ft.row_bytes("Q8_1", k)), dtype=torch.uint8, device="cuda") for k in ks}
    xs = {(k, t): xall[k][row0[t]:row0[t] + t] for k in ks for t in tokens}
    xq = {(k, t): xqall[k][row0[t]:row0[t] + t] for k in ks for t in tokens}
    cases = [(fmt, n, k, t) for (fmt, n, k) in mats for t in tokens]
    ys = {c: torch.empty((c[3], c[1]), dtype=torch.float32, device="cuda") for c in cases}

    def step(j):
        """one pass of the path over every case, weight copy j"""
        for k in ks:
            ft.quantize_act("Q8_1", dxall[k], out=xqall[k])
        for (fmt, n, k, t) in cases:
            cp = dev[(fmt, n, k)]
            ft.mul_mat_vec_q(fmt, cp[j % len(cp)], n, k, "Q8_1", xq[(k, t)], t, out=ys[(fmt, n, k, t)])

    # one graph holds `copies` consecutive steps (step j reads weight copy j)
    g_steps = _graph(torch, lambda: [step(j) for j in range(copies)])
    for _ in range(max(1, args.warmup // copies)):
        g_steps.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-args.steps // copies))
    t0 = time.perf_counter()
    for _ in range(reps):
        g_steps.replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / (reps * copies)
    steps_done = reps * copies

    # per-case kernel duration: a graph of R back-to-back launches of that case's
    # matvec over the rotating copies; the median of 7 replays, each timed with two
    # events on the launch stream
    wbytes = {c: mats[c[:3]].nbytes for c in cases}
    abytes = {c: c[3] * ft.row_bytes("Q8_1", c[2]) + 4 * c[3] * c[1] for c in cases}
    per_case, kus = [], {}
    for c in cases:
        fmt, n, k, t = c
        cp = dev[(fmt, n, k)]
        R = 8 * len(cp)
        gk = _graph(torch, lambda: [ft.mul_mat_vec_q(fmt, cp[i % len(cp)], n, k, "Q8_1",
                                                     xq[(k, t)], t, out=ys[c]) for i in range(R)])
        us = _time_graph_median(torch, gk) / R * 1e6
        kus[c] = us
        alg = wbytes[c] + abytes[c]
        per_case.append({"case": f"{fmt} {n}x{k} t={t}", "kernel_us": round(us, 2),
                         "weight_GBps": round(wbytes[c] / us / 1e3, 1),
                         "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4)})
        del gk
    head = cases.index(("Q4_K", 14336, 4096, 1)) if ("Q4_K", 14336, 4096, 1) in cases else 0
    hc = cases[head]
    h_us = kus[hc]
    h_alg = wbytes[hc] + abytes[hc]
    achieved = h_alg / h_us / 1e3
    total_w = sum(wbytes.values())
    out = {
        "metric": "Q-matvec effective weight GB/s",
        "value": round(total_w / sec / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps_done, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("i8 x i8 -> i32 (v_dot4 ring at 1 token and on 4096-long rows up to 4 tokens; int8 MFMA at "
                  "8 tokens and on 14336-long rows from 2 tokens, Q8_0 from 3), f32 scale combine"),
        "data": "synthetic (seeded GGUF blocks, N(0,1) activations)",
        "config": {"workload": (f"decode matvec, every weight format ({'/'.join(cfg['formats'])}), "
                                "W 14336x4096" if fmts_only else
                                "dense decode matvec: Q8_0 and Q4_K, W 14336x4096 and 4096x14336")
                               + f", batch {'/'.join(map(str, tokens))}, Q8_1 activations; step = one Q8_1 "
                               "quantize launch per K (all token counts' rows) + the matvec of every case, "
                               "replayed as a HIP graph",
                   "cases": len(cases),
                   "weight_copies_per_matrix": {f"{f} {n}x{k}": c for (f, n, k), c in ncp.items()},
                   "weight_bytes_per_step": total_w},
        "roofline": {"bound": "hbm", "kernel": f"mmvq {hc[0]} {hc[1]}x{hc[2]} t={hc[3]}",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic("mmvq_q4k_14336x4096_t1"),
                     "kernel_us": round(h_us, 3), "alg_bytes_per_launch": h_alg},
        "cases": per_case,
    }
    _add_ceilings(out, torch, ft)
    if not fmts_only and not args.dense_only:
        # the rest of the metric: routed-MoE layer tokens/s and the grouped GEMM
        del dev, dxall, xqall, xq, ys, g_steps
        torch.cuda.empty_cache()
        out["moe_q4k"] = moe_results(args, np, torch, ft, synth, synth.MOE_Q4K, list(synth.MOE_Q4K["tokens"]))
        torch.cuda.empty_cache()
        out["moe_mxfp4"] = moe_results(args, np, torch, ft, synth, synth.MOE_MXFP4, list(synth.MOE_MXFP4["tokens"]))
        torch.cuda.empty_cache()
        out["grouped_kq"] = grouped_results(args, np, torch, ft, synth)
        torch.cuda.empty_cache()
        out["moe_kq_layer"] = moe_results(args, np, torch, ft, synth, synth.MOE_KQ_LAYER,
                                          list(synth.MOE_KQ_LAYER["tokens"]))
    if not args.no_cpu_baseline and not fmts_only:
        import oracle
        xqs = {key: oracle.quantize("Q8_1", v) for key, v in xs.items()}

        def run():
            for (fmt, n, k, t) in cases:
                oracle.matvec(fmt, mats[(fmt, n, k)], n, k, "Q8_1", xqs[(k, t)], t)
        out["cpu_baseline"] = _cpu_baseline(run, "one full pass over the 16 dense-decode cases (all rows)",
                                            "GB/s", total_w / 1e9)
    return out


# ---------------------------------------------------------------------------
# Q4_0 2048x2048 dequant + single-token matvec
# ---------------------------------------------------------------------------
def bench_q4_0(args, np, torch, ft, synth):
    c = synth.Q4_0_MATVEC
    n, k = c["n"], c["k"]
    g = synth.rng(7, 0)
    W = synth.weights("Q4_0", n, k, g)
    copies = args.copies or 256          # 2.36 MB each: 600 MB rotated
    dW = torch.from_numpy(W).cuda()
    dWs = [dW] + [dW.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.activations(1, k, g)).cuda()
    xq = torch.empty((1, ft.row_bytes("Q8_1", k)), dtype=torch.uint8, device="cuda")
    y = torch.empty((1, n), device="cuda")
    deq = torch.empty((n, k), device="cuda")
    R = 64

    def steps():
        for j in range(R):
            ft.quantize_act("Q8_1", x, out=xq)
            ft.mul_mat_vec_q("Q4_0", dWs[j % copies], n, k, "Q8_1", xq, 1, out=y)
            ft.dequant("Q4_0", dWs[j % copies], n, k, out=deq)

    gs = _graph(torch, steps)
    sec = _time_graph(torch, gs, max(1, args.steps // R)) / R
    gm = _graph(torch, lambda: [ft.mul_mat_vec_q("Q4_0", dWs[j % copies], n, k, "Q8_1", xq, 1, out=y)
                                for j in range(R)])
    us = _time_graph_median(torch, gm) / R * 1e6
    gd = _graph(torch, lambda: [ft.dequant("Q4_0", dWs[j % copies], n, k, out=deq) for j in range(R)])
    dus = _time_graph_median(torch, gd) / R * 1e6
    alg = W.nbytes + ft.row_bytes("Q8_1", k) + 4 * n
    out = {
        "metric": "Q-matvec effective weight GB/s", "value": round(W.nbytes / sec / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": R * max(1, args.steps // R), "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 dot4 -> i32, f32 scale combine", "data": "synthetic",
        "config": {"workload": "Q4_0 2048x2048: Q8_1 quantize + single-token matvec + dequant, HIP graph",
                   "weight_copies": copies},
        "roofline": {"bound": "hbm", "kernel": "mmvq Q4_0 2048x2048 t=1", "achieved": round(alg / us / 1e3, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel_us": round(us, 3), "alg_bytes_per_launch": alg,
                     "dequant_us": round(dus, 3),
                     "dequant_GBps": round((W.nbytes + 4 * n * k) / dus / 1e3, 1)},
    }
    _add_ceilings(out, torch, ft)
    if not args.no_cpu_baseline:
        import oracle
        xqn = oracle.quantize("Q8_1", x.cpu().numpy())
        out["cpu_baseline"] = _cpu_baseline(lambda: oracle.matvec("Q4_0", W, n, k, "Q8_1", xqn, 1),
                                            "single-token Q4_0 2048x2048 matvec", "GB/s", W.nbytes / 1e9)
    return out


# ---------------------------------------------------------------------------
# routed MoE layer, tokens/s
# ---------------------------------------------------------------------------
def moe_results(args, np, torch, ft, synth, c, tokens, route=0):
    """Layer time per token count: a HIP graph of 2 x (layer banks) steps, each
    route (fresh logits) + the layer, each on another copy of the expert banks."""
    fmt, act, H, I, E, topk = c["fmt"], c["act"], c["hidden"], c["inter"], c["n_expert"], c["topk"]
    g = synth.rng(7, {"Q4_K": 3, "MXFP4": 5}.get(fmt, 6), H)
    wg = synth.expert_bank(fmt, E, I, H, g)
    wu = synth.expert_bank(fmt, E, I, H, g)
    wd = synth.expert_bank(fmt, E, H, I, g)
    layer_bytes = wg.nbytes + wu.nbytes + wd.nbytes
    layers = args.copies or max(2, min(8, int(-(-(2 << 30) // layer_bytes))))
    banks = [(torch.from_numpy(wg).cuda(), torch.from_numpy(wu).cuda(), torch.from_numpy(wd).cuda())]
    del wg, wu, wd
    for _ in range(layers - 1):
        banks.append(tuple(b.clone() for b in banks[0]))
    per_expert = layer_bytes // E
    results = []
    G = 2 * layers                       # steps per graph: each reads another layer's bank
    for t in tokens:
        x = torch.from_numpy(synth.activations(t, H, g)).cuda()
        logits = torch.from_numpy(np.stack([synth.logits(t, E, g) for _ in range(G)])).cuda()
        ids = torch.empty((G, t, topk), dtype=torch.int32, device="cuda")
        w = torch.empty((G, t, topk), dtype=torch.float32, device="cuda")
        y = torch.empty((t, H), device="cuda")
        ft.scratch_reserve(ft.moe_scratch_bytes(fmt, act, E, H, I, t, topk))

        def steps():
            # the layer routes from the step's logits itself (ids / w come back as outputs)
            for i in range(G):
                wgb, wub, wdb = banks[i % layers]
                ft.moe_q_vec(fmt, wgb, wub, wdb, E, H, I, act, x, None, None, out=y, route=route, logits=logits[i],
                             topk=topk, ids_out=ids[i], w_out=w[i])

        gs = _graph(torch, steps)
        sec = _time_graph(torch, gs, max(1, args.steps // G)) / G
        idh = ids.cpu().numpy()
        u = float(np.mean([len(np.unique(idh[i])) for i in range(G)]))
        direct_ok = (fmt, act) in (("Q4_K", "Q8_1"), ("MXFP4", "Q8_K"))
        tiles = route == 2 or (route == 0 and (not direct_ok or t > 8))
        results.append({"tokens": t, "route": "sorted tiles" if tiles else "direct",
                        "tok_per_s": round(t / sec, 1), "layer_us": round(sec * 1e6, 2),
                        "unique_experts": round(u, 2),
                        "weight_GBps": round(u * per_expert / sec / 1e9, 1),
                        "hbm_frac": round(u * per_expert / sec / 1e9 / HBM_PEAK_GBS, 4)})
        del gs, x, logits, ids, w, y
    del banks
    return {"workload": f"routed MoE layer {fmt} x {act}: hidden {H}, {E} experts of {I}, top-{topk}; step = "
                        "one ft_moe_q_vec call from the router logits (route, quantize, gate/up+SwiGLU, quantize h, "
                        "down, combine), HIP graph",
            "metric": "routed-MoE layer tokens/s", "dtype": MOE_DTYPE, "layer_banks": layers,
            "per_tokens": results}


def bench_moe(args, np, torch, ft, synth):
    c = {"moe_q4k": synth.MOE_Q4K, "moe_mxfp4": synth.MOE_MXFP4, "moe_kq_layer": synth.MOE_KQ_LAYER}[args.workload]
    tokens = [int(x) for x in args.tokens.split(",")] if args.tokens else list(c["tokens"])
    r = moe_results(args, np, torch, ft, synth, c, tokens, route=args.route)
    head = r["per_tokens"][0]
    out = {
        "metric": "routed-MoE layer tokens/s", "value": head["tok_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["layer_us"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": MOE_DTYPE, "data": "synthetic (router logits redrawn every step)",
        "config": {"workload": r["workload"], "tokens": tokens, "layer_banks": r["layer_banks"]},
        "roofline": {"bound": "hbm", "kernel": "whole MoE layer (unique experts' weight bytes / layer time)",
                     "achieved": head["weight_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["hbm_frac"], "traffic": None},
        "per_tokens": r["per_tokens"],
    }
    return _add_ceilings(out, torch, ft)


# ---------------------------------------------------------------------------
# grouped keep-quant expert GEMM, 512 tokens
# ---------------------------------------------------------------------------
def grouped_results(args, np, torch, ft, synth):
    """Each grouped GEMM case (sort + GEMM per call) in a HIP graph over 4 weight
    copies and 4 routings."""
    c = synth.GROUPED_KQ
    T, H, I, E, topk = c["tokens"], c["hidden"], c["inter"], c["n_expert"], c["topk"]
    g = synth.rng(7, 4)
    results = []
    for fmt in c["formats"]:
        for proj in ("gate_up", "down"):
            n, k = (I, H) if proj == "gate_up" else (H, I)
            W = synth.expert_bank(fmt, E, n, k, g)
            copies = args.copies or 4
            dW = torch.from_numpy(W).cuda()
            dWs = [dW] + [dW.clone() for _ in range(copies - 1)]
            per_pair = proj == "down"
            x = torch.from_numpy(synth.activations(T * topk if per_pair else T, k, g)).cuda()
            xq = ft.quantize_act("Q8_K", x)
            ids_pool = [torch.from_numpy(synth.expert_ids(T, E, topk, g)).cuda() for _ in range(copies)]
            y = torch.empty((T * topk, n), device="cuda")
            ft.scratch_reserve(1 << 20)
            gg = _graph(torch, lambda: [ft.grouped_gemm_q(fmt, dWs[i], E, n, k, "Q8_K", xq, per_pair, ids_pool[i],
                                                          out=y) for i in range(copies)])
            us = _time_graph(torch, gg, max(1, args.steps // copies)) / copies * 1e6
            ops = 2.0 * T * topk * n * k
            alg = W.nbytes + xq.numel() + y.numel() * 4
            results.append({"case": f"{fmt} {proj} {n}x{k}", "us": round(us, 2),
                            "weight_GBps": round(W.nbytes / us / 1e3, 1),
                            "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
                            "int8_TOPS": round(ops / us / 1e6, 2),
                            "mfma_frac": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4)})
            del dWs, dW, gg, W, x, xq, y
    return {"workload": f"grouped keep-quant GEMM: {T} tokens, hidden {H}, {E} experts of {I}, top-{topk}, "
                        "Q5_K/Q6_K x Q8_K (sort + GEMM per call), HIP graph",
            "cases": results}


def bench_grouped(args, np, torch, ft, synth):
    r = grouped_results(args, np, torch, ft, synth)
    head = r["cases"][0]
    out = {
        "metric": "grouped expert GEMM int8 TOP/s", "value": head["int8_TOPS"], "unit": "TOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["us"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 on int8 MFMA, f32 scale combine", "data": "synthetic",
        "config": {"workload": r["workload"]},
        "roofline": {"bound": "hbm", "kernel": head["case"], "achieved": round(head["hbm_frac"] * HBM_PEAK_GBS, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["hbm_frac"], "traffic": None},
        "cases": r["cases"],
    }
    return _add_ceilings(out, torch, ft, tops=head["int8_TOPS"])


# ---------------------------------------------------------------------------
# counter runs: a device copy of known size (calibration) and the headline kernel
# ---------------------------------------------------------------------------
def run_counters(args, np, torch, ft, synth):
    """The counter workload: calibration copies, then the headline matvec, the Q4_K
    MoE layer at 1 and 4 tokens, the MXFP4 MoE layer at 1 token and the Q5_K grouped
    GEMM (each kernel is named apart in the counter CSVs)."""
    a = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    n, k = 14336, 4096
    g = synth.rng(7, 1)
    W = torch.from_numpy(synth.weights("Q4_K", n, k, g)).cuda()
    Ws = [W] + [W.clone() for _ in range(7)]
    xq = ft.quantize_act("Q8_1", torch.from_numpy(synth.activations(1, k, g)).cuda())
    y = torch.empty((1, n), device="cuda")
    for i in range(20):
        ft.mul_mat_vec_q("Q4_K", Ws[i % 8], n, k, "Q8_1", xq, 1, out=y)
    torch.cuda.synchronize()
    del Ws, W
    if args.counters_scope == "headline":
        return {"counters_run": "copy 256 MiB x3, mmvq Q4_K 14336x4096 t=1 x20"}
    # routed MoE layers from router logits (two bank copies, so each call reads HBM)
    for c, tokens, reps in ((synth.MOE_Q4K, (1, 4), 8), (synth.MOE_MXFP4, (1,), 4)):
        fmt, act, H, I, E, topk = c["fmt"], c["act"], c["hidden"], c["inter"], c["n_expert"], c["topk"]
        gg = synth.rng(8, E)
        bank = [torch.from_numpy(synth.expert_bank(fmt, E, I, H, gg)).cuda(),
                torch.from_numpy(synth.expert_bank(fmt, E, I, H, gg)).cuda(),
                torch.from_numpy(synth.expert_bank(fmt, E, H, I, gg)).cuda()]
        banks = [bank, [t.clone() for t in bank]] if fmt == "Q4_K" else [bank]
        for t in tokens:
            x = torch.from_numpy(synth.activations(t, H, gg)).cuda()
            yy = torch.empty((t, H), device="cuda")
            for i in range(reps):
                lg = torch.from_numpy(synth.logits(t, E, gg)).cuda()
                ft.moe_q_vec(fmt, *banks[i % len(banks)], E, H, I, act, x, None, None, out=yy, logits=lg, topk=topk)
            torch.cuda.synchronize()
        del banks, bank
    # grouped GEMM, Q5_K gate-shaped bank (one projection, sort + GEMM per call)
    c = synth.GROUPED_KQ
    T, H, I, E, topk = c["tokens"], c["hidden"], c["inter"], c["n_expert"], c["topk"]
    gg = synth.rng(9)
    Wg = torch.from_numpy(synth.expert_bank("Q5_K", E, I, H, gg)).cuda()
    Wgs = [Wg, Wg.clone()]
    xg = ft.quantize_act("Q8_K", torch.from_numpy(synth.activations(T, H, gg)).cuda())
    yg = torch.empty((T * topk, I), device="cuda")
    for i in range(4):
        ids = torch.from_numpy(synth.expert_ids(T, E, topk, gg)).cuda()
        ft.grouped_gemm_q("Q5_K", Wgs[i % 2], E, I, H, "Q8_K", xg, False, ids, out=yg)
    torch.cuda.synchronize()
    return {"counters_run": "copy 256 MiB x3, mmvq Q4_K 14336x4096 t=1 x20, MoE Q4_K t=1 x8 and t=4 x8, "
                            "MoE MXFP4 t=1 x4, grouped Q5_K 512 tokens x4"}


def counters_summary(csvs):
    """Per-kernel means of every counter in rocprofv3 --pmc CSVs of `--workload
    counters` (FETCH_SIZE / WRITE_SIZE scaled by the calibration copies, in MB per
    dispatch); markdown on stdout."""
    import csv
    import statistics
    per = {}
    scale = {}
    for path in csvs:
        rs = list(csv.DictReader(open(path)))
        for cname in ("FETCH_SIZE", "WRITE_SIZE"):
            cp = sorted((r for r in rs if r["Counter_Name"] == cname and "copyBuffer" in r["Kernel_Name"]),
                        key=lambda r: int(r["Dispatch_Id"]))[:3]
            if cp:
                scale[cname] = COPY_BYTES / (statistics.median(float(r["Counter_Value"]) for r in cp) * 1024)
        for r in rs:
            per.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    names = sorted({kn for kn, _ in per})
    counters = sorted({cn for _, cn in per})
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---:|" + "---:|" * len(counters))
    for kn in names:
        if "copyBuffer" in kn or "elementwise" in kn:
            continue
        cells, nd = [], 0
        for cn in counters:
            vs = per.get((kn, cn))
            if not vs:
                cells.append("")
                continue
            nd = max(nd, len(vs))
            m = statistics.mean(vs)
            if cn in scale:
                cells.append(f"{m * 1024 * scale[cn] / 1e6:.3f} MB")
            else:
                cells.append(f"{m:.4g}")
        short = kn if len(kn) < 90 else kn[:87] + "..."
        print(f"| `{short}` | {nd} | " + " | ".join(cells) + " |")
    print()
    print("scales: " + ", ".join(f"{k} x{v:.4f}" for k, v in scale.items()))


def traffic_from(fetch_csv, write_csv):
    import csv
    import statistics

    def rows(path, counter):
        return [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]

    def calib(rs):
        # run_counters issues the three 256 MiB calibration copies before anything
        # else that copies (the weight clones come after them)
        cp = sorted((r for r in rs if "copyBuffer" in r["Kernel_Name"]), key=lambda r: int(r["Dispatch_Id"]))
        return [float(r["Counter_Value"]) for r in cp[:3]]

    rf, rw = rows(fetch_csv, "FETCH_SIZE"), rows(write_csv, "WRITE_SIZE")
    copy_f, copy_w = calib(rf), calib(rw)
    f = {}
    w = {}
    for r in rf:
        f.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    for r in rw:
        w.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    # counters report KiB; the copy reads and writes COPY_BYTES each
    fscale = COPY_BYTES / (statistics.median(copy_f) * 1024)
    wscale = COPY_BYTES / (statistics.median(copy_w) * 1024)
    mf = [v for kname, vs in f.items() if "mmvq" in kname for v in vs]
    mw = [v for kname, vs in w.items() if "mmvq" in kname for v in vs]
    fetch = statistics.mean(mf) * 1024 * fscale
    write = statistics.mean(mw) * 1024 * wscale
    try:
        d = json.load(open(TRAFFIC_PATH))
    except (OSError, ValueError):
        d = {}
    d["mmvq_q4k_14336x4096_t1"] = {"bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
                                   "write_bytes": round(write), "fetch_scale": round(fscale, 4),
                                   "write_scale": round(wscale, 4), "launches": len(mf),
                                   "src_hash": _src_hash()}
    os.makedirs(os.path.dirname(TRAFFIC_PATH), exist_ok=True)
    json.dump(d, open(TRAFFIC_PATH, "w"), indent=1)
    print(json.dumps(d["mmvq_q4k_14336x4096_t1"]))


if __name__ == "__main__":
    main()
