#!/usr/bin/env python3
"""Benchmark of the block-quantized matvec / routed-MoE path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The default workload is the dense decode matvec the
metric is quoted on: Q8_0 and Q4_K weights, W 14336x4096 and 4096x14336, batches
of 1/2/4/8 tokens, activations quantized to Q8_1.  One step is one pass of the
whole path (activation quantize + quantized matvec) over all 16 cases.  Weights
are resident in HBM before timing; every case rotates over enough distinct
weight copies that no launch can be served from the 256 MB last-level cache.

Other workloads (--workload): q4_0_matvec, moe_q4k, moe_mxfp4, grouped_kq.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense_decode",
                    choices=["dense_decode", "q4_0_matvec", "moe_q4k", "moe_mxfp4", "grouped_kq"])
    ap.add_argument("--copies", type=int, default=0, help="weight copies per matrix (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=str, default="", help="comma list overriding the token counts")
    return ap.parse_args()


def main():
    args = _args()
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
    fn = {"dense_decode": bench_dense, "q4_0_matvec": bench_q4_0, "moe_q4k": bench_moe,
          "moe_mxfp4": bench_moe, "grouped_kq": bench_grouped}[args.workload]
    out = fn(args, np, torch, ft, synth)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
class Timer:
    """Per-launch HIP events on the launching (current) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, key):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, key, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.setdefault(key, []).append((e0, e1))

    def times_us(self, key):
        return sorted(1000.0 * a.elapsed_time(b) for a, b in self.pairs.get(key, []))

    def avg_us(self, key):
        ts = self.times_us(key)
        return sum(ts) / max(len(ts), 1)

    def median_us(self, key):
        ts = self.times_us(key)
        return ts[len(ts) // 2] if ts else 0.0


def _cpu_baseline(fn, sample_desc, unit, work):
    import oracle
    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"value": work / dt, "unit": unit, "cores": oracle.threads(), "kind": "oracle",
            "sample": sample_desc, "seconds": round(dt, 3)}


def _timed(torch, steps, warmup, step_fn, timer=None):
    for i in range(warmup):
        step_fn(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_fn(warmup + i, timer)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


# ---------------------------------------------------------------------------
# dense decode matvec (the headline workload)
# ---------------------------------------------------------------------------
def bench_dense(args, np, torch, ft, synth):
    cfg = synth.DENSE_DECODE
    tokens = [int(x) for x in args.tokens.split(",")] if args.tokens else list(cfg["tokens"])
    g = synth.rng(7, 1)
    mats = {}
    for fmt in cfg["formats"]:
        for (n, k) in cfg["shapes"]:
            W = synth.weights(fmt, n, k, g)
            mats[(fmt, n, k)] = W
    # each matrix is used once per token count per step and every use takes the
    # next copy: with 8 copies, >= 1.5 GB of other weights stream between two
    # uses of one copy (the last-level cache is 256 MB)
    total = sum(W.nbytes for W in mats.values())
    copies = args.copies or 8
    dev = {key: [torch.from_numpy(W).cuda()] for key, W in mats.items()}
    for key in dev:
        base = dev[key][0]
        dev[key] += [base.clone() for _ in range(copies - 1)]
    xs = {(k, t): synth.activations(t, k, g) for (_, _, k) in mats for t in tokens}
    dxs = {key: torch.from_numpy(v).cuda() for key, v in xs.items()}
    xq = {(k, t): torch.empty((t, ft.row_bytes("Q8_1", k)), dtype=torch.uint8, device="cuda")
          for (k, t) in xs}
    cases = [(fmt, n, k, t) for (fmt, n, k) in mats for t in tokens]
    ys = {c: torch.empty((c[3], c[1]), dtype=torch.float32, device="cuda") for c in cases}
    use = {}

    def step(i, timer):
        for ci, (fmt, n, k, t) in enumerate(cases):
            j = use.get((fmt, n, k), 0)
            use[(fmt, n, k)] = (j + 1) % copies
            ft.quantize_act("Q8_1", dxs[(k, t)], out=xq[(k, t)])
            e0 = timer.start(ci) if timer else None
            ft.mul_mat_vec_q(fmt, dev[(fmt, n, k)][j], n, k, "Q8_1", xq[(k, t)], t, out=ys[(fmt, n, k, t)])
            if timer:
                timer.stop(ci, e0)

    timer = Timer(torch)
    sec = _timed(torch, args.steps, args.warmup, step, timer)
    wbytes = {c: mats[c[:3]].nbytes for c in cases}
    abytes = {c: c[3] * ft.row_bytes("Q8_1", c[2]) + 4 * c[3] * c[1] for c in cases}
    per_case = []
    for ci, c in enumerate(cases):
        us = timer.avg_us(ci)
        alg = wbytes[c] + abytes[c]
        per_case.append({"case": f"{c[0]} {c[1]}x{c[2]} t={c[3]}", "kernel_us": round(us, 2),
                         "median_us": round(timer.median_us(ci), 2),
                         "weight_GBps": round(wbytes[c] / us / 1e3, 1),
                         "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4)})
    head = cases.index(("Q4_K", 14336, 4096, 1)) if ("Q4_K", 14336, 4096, 1) in cases else 0
    hc = cases[head]
    h_us = timer.avg_us(head)
    h_alg = wbytes[hc] + abytes[hc]
    achieved = h_alg / h_us / 1e3
    total_w = sum(wbytes.values())
    out = {
        "metric": "Q-matvec effective weight GB/s",
        "value": round(total_w / sec / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 dot4 -> i32, f32 scale combine",
        "data": "synthetic (seeded GGUF blocks, N(0,1) activations)",
        "config": {"workload": "dense decode matvec: Q8_0 and Q4_K, W 14336x4096 and 4096x14336, "
                               f"batch {'/'.join(map(str, tokens))}, Q8_1 activations; step = quantize + "
                               "matvec for all cases",
                   "cases": len(cases), "weight_copies_per_matrix": copies,
                   "weight_bytes_per_step": total_w},
        "roofline": {"bound": "hbm", "kernel": f"mmvq {hc[0]} {hc[1]}x{hc[2]} t={hc[3]}",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_us": round(h_us, 3), "alg_bytes_per_launch": h_alg},
        "cases": per_case,
    }
    if not args.no_cpu_baseline:
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
    copies = args.copies or 1024
    dW = torch.from_numpy(W).cuda()
    dWs = [dW] + [dW.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.activations(1, k, g)).cuda()
    xq = torch.empty((1, ft.row_bytes("Q8_1", k)), dtype=torch.uint8, device="cuda")
    y = torch.empty((1, n), device="cuda")
    deq = torch.empty((n, k), device="cuda")

    def step(i, timer):
        Wc = dWs[i % copies]
        ft.quantize_act("Q8_1", x, out=xq)
        e0 = timer.start("mmvq") if timer else None
        ft.mul_mat_vec_q("Q4_0", Wc, n, k, "Q8_1", xq, 1, out=y)
        if timer:
            timer.stop("mmvq", e0)
            e1 = timer.start("deq")
        ft.dequant("Q4_0", Wc, n, k, out=deq)
        if timer:
            timer.stop("deq", e1)

    timer = Timer(torch)
    sec = _timed(torch, args.steps, args.warmup, step, timer)
    us = timer.avg_us("mmvq")
    alg = W.nbytes + ft.row_bytes("Q8_1", k) + 4 * n
    out = {
        "metric": "Q-matvec effective weight GB/s", "value": round(W.nbytes / sec / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 dot4 -> i32, f32 scale combine", "data": "synthetic",
        "config": {"workload": "Q4_0 2048x2048: Q8_1 quantize + dequant + single-token matvec",
                   "weight_copies": copies},
        "roofline": {"bound": "hbm", "kernel": "mmvq Q4_0 2048x2048 t=1", "achieved": round(alg / us / 1e3, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel_us": round(us, 3), "alg_bytes_per_launch": alg,
                     "dequant_us": round(timer.avg_us("deq"), 3)},
    }
    if not args.no_cpu_baseline:
        import oracle
        xqn = oracle.quantize("Q8_1", x.cpu().numpy())

        def run():
            for _ in range(20):
                oracle.matvec("Q4_0", W, n, k, "Q8_1", xqn, 1)
        out["cpu_baseline"] = _cpu_baseline(run, "20 single-token Q4_0 2048x2048 matvecs", "GB/s",
                                            20 * W.nbytes / 1e9)
    return out


# ---------------------------------------------------------------------------
# routed MoE vector layer (direct route), tokens/s
# ---------------------------------------------------------------------------
def bench_moe(args, np, torch, ft, synth):
    c = synth.MOE_Q4K if args.workload == "moe_q4k" else synth.MOE_MXFP4
    fmt, act, H, I, E, topk = c["fmt"], c["act"], c["hidden"], c["inter"], c["n_expert"], c["topk"]
    tokens = [int(x) for x in args.tokens.split(",")] if args.tokens else [t for t in c["tokens"] if t <= 4]
    g = synth.rng(7, 3 if fmt == "Q4_K" else 5)
    wg = synth.expert_bank(fmt, E, I, H, g)
    wu = synth.expert_bank(fmt, E, I, H, g)
    wd = synth.expert_bank(fmt, E, H, I, g)
    layer_bytes = wg.nbytes + wu.nbytes + wd.nbytes
    layers = args.copies or max(2, min(8, int(-(-(2 << 30) // layer_bytes))))
    banks = [(torch.from_numpy(wg).cuda(), torch.from_numpy(wu).cuda(), torch.from_numpy(wd).cuda())]
    for _ in range(layers - 1):
        banks.append(tuple(b.clone() for b in banks[0]))
    per_expert = layer_bytes // E
    results = []
    steps_logits = args.steps + args.warmup
    for t in tokens:
        x = torch.from_numpy(synth.activations(t, H, g)).cuda()
        logits = torch.from_numpy(np.stack([synth.logits(t, E, g) for _ in range(steps_logits)])).cuda()
        y = torch.empty((t, H), device="cuda")
        ft.scratch_reserve(ft.moe_scratch_bytes(fmt, act, E, H, I, t, topk))
        uniq = []

        def step(i, timer):
            wgb, wub, wdb = banks[i % layers]
            ids, w = ft.moe_route(logits[i], topk)
            e0 = timer.start("layer") if timer else None
            ft.moe_q_vec(fmt, wgb, wub, wdb, E, H, I, act, x, ids, w, out=y)
            if timer:
                timer.stop("layer", e0)
                uniq.append(ids)

        timer = Timer(torch)
        sec = _timed(torch, args.steps, args.warmup, step, timer)
        u = np.mean([len(np.unique(i.cpu().numpy())) for i in uniq])
        us = timer.avg_us("layer")
        results.append({"tokens": t, "tok_per_s": round(t / sec, 1), "layer_us": round(sec * 1e6, 2),
                        "moe_vec_us": round(us, 2), "unique_experts": round(float(u), 2),
                        "weight_GBps": round(u * per_expert / us / 1e3, 1),
                        "hbm_frac": round(u * per_expert / us / 1e3 / HBM_PEAK_GBS, 4)})
    head = results[0]
    out = {
        "metric": "routed-MoE layer tokens/s", "value": head["tok_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["layer_us"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 dot4 -> i32, f32 scale combine", "data": "synthetic (router logits redrawn every step)",
        "config": {"workload": f"routed MoE layer {fmt} x {act}: hidden {H}, {E} experts of {I}, top-{topk}, "
                               f"direct route; step = route + quantize + gate/up+SwiGLU + quantize + down + combine",
                   "tokens": tokens, "layer_banks": layers},
        "roofline": {"bound": "hbm", "kernel": "moe_q_vec (all stages)", "achieved": head["weight_GBps"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["hbm_frac"], "traffic": None},
        "per_tokens": results,
    }
    return out


# ---------------------------------------------------------------------------
# grouped keep-quant expert GEMM, 512 tokens
# ---------------------------------------------------------------------------
def bench_grouped(args, np, torch, ft, synth):
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
            ids_pool = [torch.from_numpy(synth.expert_ids(T, E, topk, g)).cuda() for _ in range(4)]
            y = torch.empty((T * topk, n), device="cuda")
            ft.scratch_reserve(1 << 20)

            def step(i, timer):
                e0 = timer.start("g") if timer else None
                ft.grouped_gemm_q(fmt, dWs[i % copies], E, n, k, "Q8_K", xq, per_pair, ids_pool[i % 4], out=y)
                if timer:
                    timer.stop("g", e0)

            timer = Timer(torch)
            _timed(torch, args.steps, args.warmup, step, timer)
            us = timer.avg_us("g")
            ops = 2.0 * T * topk * n * k
            alg = W.nbytes + xq.numel() + y.numel() * 4
            results.append({"case": f"{fmt} {proj} {n}x{k}", "us": round(us, 2),
                            "hbm_frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4),
                            "int8_TOPS": round(ops / us / 1e6, 2),
                            "mfma_frac": round(ops / us / 1e6 / INT8_PEAK_TOPS, 4)})
            del dWs, dW
    head = results[0]
    out = {
        "metric": "grouped expert GEMM int8 TOP/s", "value": head["int8_TOPS"], "unit": "TOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["us"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 dot4 -> i32, f32 scale combine", "data": "synthetic",
        "config": {"workload": f"grouped keep-quant GEMM: {T} tokens, hidden {H}, {E} experts of {I}, "
                               f"top-{topk}, Q5_K/Q6_K x Q8_K"},
        "roofline": {"bound": "hbm", "kernel": head["case"], "achieved": round(head["hbm_frac"] * HBM_PEAK_GBS, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["hbm_frac"], "traffic": None},
        "cases": results,
    }
    return out


if __name__ == "__main__":
    main()
