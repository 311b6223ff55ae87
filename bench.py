#!/usr/bin/env python3
"""Benchmark of the Q6_K MMVQ decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]

Workload (one "step"): quantize 13 fp32 activation columns to Q8_1 (the
column-planar arrangement of its bytes) in one launch, then run the Q6_K
MMVQ of a 10240 x 2560 (rows x cols) matrix in the tiled layout (int8
matrix-core kernel) at N = 1, 4 and 8 columns (each product on its own
columns: 1 + 4 + 8 = 13)
-- the decode matrix the pages measure as "2560 x 10240" (n_in x n_out).  Weights are resident in HBM before timing and
each launch reads a different one of 26 copies (559 MB, more than twice the
256 MB Infinity Cache), so every weight byte comes from HBM.

Printed: one JSON line.  `value` is effective weight throughput over the
whole step (weight bytes of the three products / step wall time, GB/s).
`roofline` is for the dominant kernel (the MMVQ instantiation with the
largest share of GPU time): algorithmic bytes per launch over its average
launch time, from HIP events on its launch stream around graph replays of
back-to-back launches.  The step itself is timed from HIP graph replays,
each graph holding 26 consecutive steps (events on the stream, and host wall
time; the larger is used); `extras` also gives the rate with one graph launch
per step.  `cpu_baseline` times the CPU oracle on
the same step.  `extras` holds per-N figures, the other shapes, the grouped
MoE, a cache-warm figure (not HBM) and a plain device copy for calibration.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROWS, K = 10240, 2560
# HBM traffic of the dominant kernel per launch, from rocprofv3 --pmc
# FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by the same counters on a
# plain copy of known size (FETCH_SIZE x 1.9977, WRITE_SIZE x 1.0); to be
# emptied whenever the kernel changes after the counters were taken.
TRAFFIC = {1: 21671450, 4: 21866882, 8: 22143231}
NCOLS = (1, 4, 8)
XCOLS = sum(NCOLS)          # distinct activation columns quantized per step
COL0 = {1: 0, 4: 1, 8: 5}   # first activation column of each product
Q6K_BYTES = 210
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2**20
# pages' figures for this matrix (Arc A770, large-GRF launch, 1/4/8 columns):
# 86.1, 92.9, 370.5 us per call
PAGES_US = {1: 86.1, 4: 92.9, 8: 370.5}


def weight_bytes(rows, k, per_block=Q6K_BYTES):
    return rows * (k // 256) * per_block


def alg_bytes(rows, k, n, per_block=Q6K_BYTES):
    """Algorithmic bytes of one MMVQ launch: weights once, Q8_1 activations,
    fp32 outputs."""
    return weight_bytes(rows, k, per_block) + n * (k // 32) * 36 + 4 * n * rows


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--pmc-workload", action="store_true",
                   help="only run 30 launches each of the N=1/4/8 products and of a 21.5 MB device "
                        "copy (for rocprofv3 --pmc passes), print nothing")
    p.add_argument("--pmc-mmq", action="store_true",
                   help="only run 8 launches of the 512-column product mmq_q6k on the same matrix "
                        "(for rocprofv3 --pmc passes), print nothing")
    return p.parse_args()


def timed_launches(torch, fn, n_iter, copies):
    """Per-launch GPU time (us) from events around each launch; fn(buf)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_iter)]
    for i in range(n_iter):
        evs[i][0].record()
        fn(copies[i % len(copies)])
        evs[i][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return {"mean_us": sum(t) / len(t), "median_us": t[len(t) // 2], "p10_us": t[len(t) // 10],
            "p90_us": t[(9 * len(t)) // 10]}


def graph_avg_us(torch, calls, reps=6):
    """Average device time per call (us): events on the current stream around
    replays of a HIP graph holding the calls back to back."""
    stream = torch.cuda.current_stream()
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph, stream=stream):
        for c in calls:
            c()
    gph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        gph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * len(calls))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this benchmark runs on one GPU only (the MMVQ would shard by output rows "
              "across GPUs; no multi-GPU path is built). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quant_mat_vec_amd import qmv, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    # all work on one non-default stream (graph capture needs one; default
    # priority, like every stream here)
    torch.cuda.set_stream(torch.cuda.Stream())
    # tiled weights (matrix cores), column-planar Q8_1 activations
    XT = qmv.LAYOUT_TILED | qmv.ACT_PLANAR
    g = synth.rng(synth.seed_for(1, 1, 8))
    w_np = synth.q6k_blocks(g, ROWS, K)
    x_np = synth.activations(g, XCOLS, K)
    wb = weight_bytes(ROWS, K)
    ncopies = max(2, math.ceil(2 * MALL_BYTES / wb) + 1)
    w_gguf = torch.from_numpy(w_np).to(dev)
    base = torch.empty_like(w_gguf)
    qmv.repack_q6k_tiled(w_gguf, base, ROWS, K)
    copies = [base.clone() for _ in range(ncopies)]
    xd = torch.from_numpy(x_np).to(dev)
    xq_all = torch.empty(XCOLS * (K // 32) * 36, dtype=torch.uint8, device=dev)
    qcol = (K // 32) * 36      # bytes of one Q8_1 column

    def xq_of(n):
        return xq_all[COL0[n] * qcol:(COL0[n] + n) * qcol]
    qmv.quantize_q8_1_planar(xd, xq_all, K, XCOLS)
    xq = xq_all[:8 * qcol]
    out = torch.empty(8 * ROWS, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    if args.pmc_mmq:
        n = 512
        xm = torch.from_numpy(synth.activations(g, n, K)).to(dev)
        qm = torch.empty(n * qcol, dtype=torch.uint8, device=dev)
        om = torch.empty(n * ROWS, dtype=torch.float32, device=dev)
        qmv.quantize_q8_1_planar(xm, qm, K, n)
        for i in range(8):
            qmv.mmq_q6k(copies[i % ncopies], XT, qm, om, ROWS, K, n)
        torch.cuda.synchronize()
        return

    if args.pmc_workload:
        # fixed workload for hardware-counter passes: the three products on
        # rotated copies, then a plain copy of the same size (its FETCH_SIZE /
        # WRITE_SIZE calibrate the counters against known bytes)
        qmv.quantize_q8_1_planar(xd, xq_all, K, XCOLS)
        for n in NCOLS:
            for i in range(30):
                qmv.mmvq_q6k(copies[i % ncopies], XT, xq_of(n), out, ROWS, K, n)
        dst = torch.empty_like(base)
        for i in range(30):
            dst.copy_(copies[i % ncopies])
        torch.cuda.synchronize()
        return

    def step(i):
        qmv.quantize_q8_1_planar(xd, xq_all, K, XCOLS)
        for j, n in enumerate(NCOLS):
            c = copies[(len(NCOLS) * i + j) % ncopies]
            qmv.mmvq_q6k(c, XT, xq_of(n), out, ROWS, K, n)

    # Step i uses weight copies at rotation offset i % ncopies.  HIP graphs:
    # one holding `ncopies` consecutive steps (offsets 0 .. ncopies-1, so the
    # rotation continues across replays) and one single-step graph per
    # offset for a remainder; exactly `steps` steps run in the timed region.
    # A decode loop captures many launches per graph; the single-step figure
    # (one graph launch per step) is reported beside it.
    graphs = []
    for i in range(ncopies):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph, stream=stream):
            step(i)
        graphs.append(gph)
    multi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi, stream=stream):
        for i in range(ncopies):
            step(i)
    torch.cuda.synchronize()

    def run_steps(n, batched):
        done = 0
        if batched:
            while n - done >= ncopies:
                multi.replay()
                done += ncopies
        while done < n:
            graphs[done % ncopies].replay()
            done += 1

    def timed_steps(n, batched):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        run_steps(n, batched)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return e0.elapsed_time(e1) / n, (t1 - t0) * 1e3 / n

    run_steps(args.warmup, True)
    torch.cuda.synchronize()
    ms_per_step, wall_ms_per_step = timed_steps(args.steps, True)
    step_bytes = wb * len(NCOLS)
    value = step_bytes / (max(ms_per_step, wall_ms_per_step) * 1e-3) / 1e9
    single_ms, single_wall_ms = timed_steps(args.steps, False)

    # Per-kernel average launch time: events on the launch stream around
    # graph replays of back-to-back launches of one MMVQ instantiation
    # (rotating copies), so host launch cost is excluded and only the device's
    # per-launch time (kernel plus the dispatch gap between kernels) remains.
    per_n = {}
    reps, per_graph = 8, ncopies * 2
    qmv.quantize_q8_1_planar(xd, xq_all, K, XCOLS)
    for n in NCOLS:
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph, stream=stream):
            for i in range(per_graph):
                qmv.mmvq_q6k(copies[i % ncopies], XT, xq_of(n), out, ROWS, K, n)
        gph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            gph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        mean = a.elapsed_time(b) * 1e3 / (reps * per_graph)
        per_n[n] = {"kernel": f"qmv::k_mmvq_q6_tiled<{n}, 4, 1, 5, false, false, true>",
                    "avg_launch_us": round(mean, 3),
                    "weight_GBps": round(wb / (mean * 1e-6) / 1e9, 1),
                    "weight_frac_of_8TBps": round(wb / (mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "alg_bytes": alg_bytes(ROWS, K, n), "launches_timed": reps * per_graph}
        del gph
    dom = max(NCOLS, key=lambda n: per_n[n]["avg_launch_us"])
    ach = alg_bytes(ROWS, K, dom) / (per_n[dom]["avg_launch_us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": TRAFFIC.get(dom),
                "kernel": per_n[dom]["kernel"], "ncols": dom,
                "alg_bytes_per_launch": alg_bytes(ROWS, K, dom),
                "avg_launch_us": per_n[dom]["avg_launch_us"]}

    # eager launches with per-launch events (host launch path included)
    eager = {}
    for n in NCOLS:
        r = timed_launches(torch, lambda c, n=n: qmv.mmvq_q6k(c, XT, xq_of(n), out, ROWS, K, n), 100, copies)
        eager[str(n)] = round(r["mean_us"], 3)

    # checksum of the last step's N=8 output bits (FNV-1a 32)
    torch.cuda.synchronize()
    ob = out.cpu().numpy().view(np.uint32)
    h = np.uint32(2166136261)
    for byte in ob.view(np.uint8)[:4096 * 4]:
        h = np.uint32((int(h) ^ int(byte)) * 16777619 & 0xFFFFFFFF)

    extras = {"per_ncols": {str(n): per_n[n] for n in NCOLS},
              "eager_event_us_per_launch": eager,
              "wall_ms_per_step": round(wall_ms_per_step, 4),
              "one_graph_launch_per_step": {"ms_per_step": round(single_ms, 4),
                                            "wall_ms_per_step": round(single_wall_ms, 4),
                                            "weight_GBps": round(step_bytes / (max(single_ms, single_wall_ms) * 1e-3) / 1e9, 1)},
              "steps_per_graph": ncopies,
              "weight_copies": ncopies, "weight_bytes_per_copy": wb,
              "fnv1a32_out_prefix": int(h),
              "pages_A770_us": PAGES_US}
    if not args.no_extras:
        extras.update(run_extras(torch, np, qmv, synth, dev, copies, base, xd, xq, out))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(np, synth, w_np, x_np, args.cpu_seconds)

    pages_gbs = step_bytes / (sum(PAGES_US.values()) * 1e-6) / 1e9
    line = {
        "metric": "Q6_K MMVQ us/call and effective weight GB/s (% HBM peak) at 1/4/8 columns",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": round(value / pages_gbs, 2), "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "Q6_K MMVQ 10240x2560 (rows x cols), tiled weights (matrix cores), 1/4/8 columns, "
                               "one Q8_1 quantize (column-planar layout) of the 13 activation columns + the three MMVQs, "
                               f"weights rotated over {ncopies} HBM copies",
                   "rows": ROWS, "cols": K, "ncols": list(NCOLS),
                   "vs_baseline_basis": f"pages' A770 large-GRF figures for this matrix "
                                        f"(86.1/92.9/370.5 us) = {pages_gbs:.1f} GB/s; other hardware, context"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line))


def run_extras(torch, np, qmv, synth, dev, copies, base, xd, xq, out):
    PL, GG, TL = qmv.LAYOUT_PLANAR, qmv.LAYOUT_GGUF, qmv.LAYOUT_TILED
    ex = {}
    it = 200
    # cache-warm: the same buffer every launch (Infinity Cache / L2 resident)
    warm = {}
    for n in NCOLS:
        qmv.quantize_q8_1(xd, xq, K, n)
        us = graph_avg_us(torch, [lambda n=n: qmv.mmvq_q6k(base, TL, xq, out, ROWS, K, n)] * 52)
        warm[str(n)] = {"avg_launch_us": round(us, 3),
                        "weight_GBps_not_hbm": round(weight_bytes(ROWS, K) / (us * 1e-6) / 1e9, 1)}
    ex["cache_warm_not_hbm"] = warm
    # plain streaming reads and a device copy of the same bytes, rotated:
    # the achievable ceiling at this size
    wb = weight_bytes(ROWS, K)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    us = graph_avg_us(torch, [lambda c=c: qmv.qmv_stream_read(c, wb // 16 * 16, sink, 0) for c in copies * 2])
    ex["stream_read_calibration"] = {"bytes": wb, "avg_launch_us": round(us, 3),
                                     "read_GBps": round(wb / (us * 1e-6) / 1e9, 1)}
    dst = torch.empty_like(base)
    us = graph_avg_us(torch, [lambda c=c: dst.copy_(c) for c in copies * 2])
    ex["copy_calibration"] = {"bytes_read": wb, "avg_launch_us": round(us, 3),
                              "read_plus_write_GBps": round(2 * wb / (us * 1e-6) / 1e9, 1)}

    def shape_case(kind, rows, k, ncols_list, layout=TL, seed=0):
        g = synth.rng(seed)
        per = {"q6k": 210, "q4k": 144, "q5k": 176}[kind]
        w = torch.from_numpy(synth.blocks(kind, g, rows, k)).to(dev)
        wbytes = weight_bytes(rows, k, per)
        if kind == "q6k" and layout != GG:
            p = torch.empty_like(w)
            (qmv.repack_q6k_planar if layout == PL else qmv.repack_q6k_tiled)(w, p, rows, k)
            w = p
        nc = max(2, math.ceil(2 * MALL_BYTES / wbytes) + 1)
        cs = [w] + [w.clone() for _ in range(nc - 1)]
        x = torch.from_numpy(synth.activations(g, max(ncols_list), k)).to(dev)
        q = torch.empty(max(ncols_list) * (k // 32) * 36, dtype=torch.uint8, device=dev)
        o = torch.empty(max(ncols_list) * rows, dtype=torch.float32, device=dev)
        res = {}
        for n in ncols_list:
            qmv.quantize_q8_1(x, q, k, n)
            if kind == "q6k":
                fn = lambda c, n=n: qmv.mmvq_q6k(c, layout, q, o, rows, k, n)  # noqa: E731
            elif kind == "q4k":
                fn = lambda c, n=n: qmv.mmvq_q4k(c, q, o, rows, k, n)  # noqa: E731
            else:
                fn = lambda c, n=n: qmv.mmvq_q5k(c, q, o, rows, k, n)  # noqa: E731
            calls = [lambda c=c, fn=fn: fn(c) for c in cs] * max(1, 40 // len(cs))
            us = graph_avg_us(torch, calls, reps=4)
            res[str(n)] = {"avg_launch_us": round(us, 3),
                           "weight_GBps": round(wbytes / (us * 1e-6) / 1e9, 1)}
        del cs
        torch.cuda.empty_cache()
        return res

    ex["q6k_10240x2560_planar_dot4"] = shape_case("q6k", 10240, 2560, (1, 2, 4, 6, 8), layout=PL, seed=12)
    ex["q6k_10240x2560_2_6cols"] = shape_case("q6k", 10240, 2560, (2, 6), seed=12)
    ex["q6k_2560x10240"] = shape_case("q6k", 2560, 10240, (1, 2, 4, 6, 8), seed=11)
    ex["q6k_2560x10240_planar_dot4"] = shape_case("q6k", 2560, 10240, (1, 2, 4, 6, 8), layout=PL, seed=11)
    ex["q6k_2560x2560"] = shape_case("q6k", 2560, 2560, (1,), seed=13)
    ex["q6k_lm_head_151936x2560"] = shape_case("q6k", 151936, 2560, (1, 4), seed=14)
    ex["q6k_lm_head_151936x2560_planar_dot4"] = shape_case("q6k", 151936, 2560, (1, 4), layout=PL, seed=14)
    ex["q6k_lm_head_151936x2560_gguf"] = shape_case("q6k", 151936, 2560, (1, 4), layout=GG, seed=14)
    ex["q6k_lm_head_argmax_and_draft_gather"] = lm_head_case(torch, np, qmv, synth, dev)
    for kind in ("q4k", "q5k"):
        for (r_, k_) in ((12288, 2560), (6144, 2560), (2560, 6144), (512, 2560)):
            ex[f"{kind}_{r_}x{k_}"] = shape_case(kind, r_, k_, (1, 4), seed=15 + r_)
    ex["moe_e128_2560_768"] = moe_case(torch, np, qmv, synth, dev)
    ex["rmsnorm_quantize_13x2560"] = norm_case(torch, np, qmv, synth, dev)
    ex["q6k_many_columns_mmq"] = {f"{r_}x{k_}": prefill_case(torch, qmv, synth, dev, r_, k_)
                                  for (r_, k_) in ((10240, 2560), (2560, 10240))}
    return ex


def prefill_case(torch, qmv, synth, dev, rows, k, ncols_list=(16, 64, 128, 512)):
    """The many-column product (mmq_q6k, column-planar activations) on tiled
    weights rotated over HBM copies: per call, the int8 multiply-adds it
    computes against the int8 matrix-core peak, and the same columns as
    decode products of eight columns for context."""
    XT = qmv.LAYOUT_TILED | qmv.ACT_PLANAR
    g = synth.rng(synth.seed_for(6, rows % 101, k % 101))
    w = torch.from_numpy(synth.q6k_blocks(g, rows, k)).to(dev)
    t0 = torch.empty_like(w)
    qmv.repack_q6k_tiled(w, t0, rows, k)
    del w
    wbytes = weight_bytes(rows, k)
    cs = [t0] + [t0.clone() for _ in range(max(1, math.ceil(2 * MALL_BYTES / wbytes)))]
    nmax = max(ncols_list)
    x = torch.from_numpy(synth.activations(g, nmax, k)).to(dev)
    q = torch.empty(nmax * (k // 32) * 36, dtype=torch.uint8, device=dev)
    o = torch.empty(nmax * rows, dtype=torch.float32, device=dev)
    qmv.quantize_q8_1_planar(x, q, k, nmax)
    cb = 36 * (k // 32)
    res = {}
    for n in ncols_list:
        us = graph_avg_us(torch, [lambda c=c, n=n: qmv.mmq_q6k(c, XT, q, o, rows, k, n) for c in cs], reps=3)
        dec = graph_avg_us(torch, [lambda c=c, n=n: [qmv.mmvq_q6k(c, XT, q[i * cb:], o[i * rows:], rows, k,
                                                                  min(8, n - i)) for i in range(0, n, 8)]
                                   for c in cs[:8]], reps=2)
        ops = 2.0 * rows * k * n
        res[str(n)] = {"avg_call_us": round(us, 3), "int8_TOPs": round(ops / (us * 1e-6) / 1e12, 1),
                       "frac_of_int8_mfma_peak": round(ops / (us * 1e-6) / 5.0e15, 4),
                       "weight_GBps": round(wbytes / (us * 1e-6) / 1e9, 1),
                       "as_8col_decode_products_us": round(dec, 3)}
    del cs
    torch.cuda.empty_cache()
    return res


def norm_case(torch, np, qmv, synth, dev):
    """The fused RMSNorm -> Q8_1 launch on the step's 13 columns: per call
    from graph replays, and eager beside an unfused form (the norm as plain
    torch ops, then quantize_q8_1) for context."""
    g = synth.rng(77)
    x = torch.from_numpy(synth.activations(g, XCOLS, K)).to(dev)
    gam = torch.from_numpy((0.5 + g.random(K)).astype(np.float32)).to(dev)
    xq = torch.empty(XCOLS * (K // 32) * 36, dtype=torch.uint8, device=dev)
    eps = 1e-6
    fused_us = graph_avg_us(torch, [lambda: qmv.rmsnorm_quantize_q8_1(x, gam, eps, xq, K, XCOLS)] * 50)

    def unfused():
        y = x * torch.rsqrt(x.pow(2).mean(dim=1, keepdim=True) + eps) * gam
        qmv.quantize_q8_1(y, xq, K, XCOLS)

    def eager_us(fn, n=200):
        for _ in range(10):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    return {"fused_graph_us": round(fused_us, 3),
            "fused_eager_us": round(eager_us(lambda: qmv.rmsnorm_quantize_q8_1(x, gam, eps, xq, K, XCOLS)), 3),
            "unfused_torch_norm_plus_quantize_eager_us": round(eager_us(unfused), 3),
            "plain_quantize_graph_us": round(graph_avg_us(torch, [lambda: qmv.quantize_q8_1(x, xq, K, XCOLS)] * 50), 3)}


def lm_head_case(torch, np, qmv, synth, dev):
    """LM head 151936x2560 (tiled): the fused greedy argmax (product with
    per-tile maxima + one reduction launch) beside the product alone, per
    call; and the load-time gather of a 32768-row draft head plus the
    product on it."""
    TL = qmv.LAYOUT_TILED
    rows, k = 151936, 2560
    g = synth.rng(synth.seed_for(2, 1, 4))
    w = torch.from_numpy(synth.q6k_blocks(g, rows, k)).to(dev)
    t0 = torch.empty_like(w)
    qmv.repack_q6k_tiled(w, t0, rows, k)
    del w
    cs = [t0, t0.clone()]                      # 638 MB: more than twice the Infinity Cache
    x = torch.from_numpy(synth.activations(g, 4, k)).to(dev)
    q = torch.empty(4 * (k // 32) * 36, dtype=torch.uint8, device=dev)
    o = torch.empty(4 * rows, dtype=torch.float32, device=dev)
    idx = torch.empty(4, dtype=torch.int32, device=dev)
    val = torch.empty(4, dtype=torch.float32, device=dev)
    res = {}
    for n in (1, 4):
        qmv.quantize_q8_1(x, q, k, n)
        nws = qmv.mmvq_q6k_argmax_workspace(rows, n)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        fused = graph_avg_us(torch, [lambda c=c, n=n: qmv.mmvq_q6k_argmax(c, TL, q, rows, k, n, idx, val, ws, nws)
                                     for c in cs] * 10, reps=4)
        product = graph_avg_us(torch, [lambda c=c, n=n: qmv.mmvq_q6k(c, TL, q, o, rows, k, n) for c in cs] * 10,
                               reps=4)
        res[f"argmax_N{n}"] = {"fused_argmax_us": round(fused, 3), "product_alone_us": round(product, 3)}
    ids = torch.from_numpy(np.sort(synth.rng(77).choice(rows, size=32768, replace=False)).astype(np.int32)).to(dev)
    dh = torch.empty(32768 * (k // 256) * 210, dtype=torch.uint8, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    qmv.gather_q6k_rows(t0, TL, rows, k, ids, 32768, dh)
    b.record()
    torch.cuda.synchronize()
    res["draft_head_gather_32768_rows_us_load_time"] = round(a.elapsed_time(b) * 1e3, 1)
    dcs = [dh] + [dh.clone() for _ in range(8)]   # 619 MB
    qmv.quantize_q8_1(x, q, k, 4)
    us = graph_avg_us(torch, [lambda c=c: qmv.mmvq_q6k(c, TL, q, o, 32768, k, 4) for c in dcs] * 4, reps=4)
    res["draft_head_32768x2560_N4_us"] = round(us, 3)
    res["draft_head_weight_GBps"] = round(32768 * 10 * 210 / (us * 1e-6) / 1e9, 1)
    del cs, dcs
    torch.cuda.empty_cache()
    return res


def moe_case(torch, np, qmv, synth, dev):
    E, DM, DFF, TOPK = 128, 2560, 768, 8
    g = synth.rng(synth.seed_for(4, 0, 0))
    gate, up, down = synth.moe_weights(g, E, DM, DFF)
    gd, ud = torch.from_numpy(gate).to(dev), torch.from_numpy(up).to(dev)
    dd = torch.from_numpy(down).to(dev)
    dp = torch.empty_like(dd)
    qmv.repack_q6k_planar(dd, dp, E * DM, DFF)
    del dd
    res = {}
    per_expert = 2 * DFF * (DM // 256) * 144 + DM * (DFF // 256) * 210
    for T in (1, 2, 4, 8):
        sets = []
        for s in range(8):                      # different routings (and so different experts)
            ids, rw = synth.routing(synth.rng(1000 + 10 * T + s), T, E, TOPK)
            x = synth.activations(synth.rng(2000 + 10 * T + s), T, DM)
            xq = torch.empty(T * (DM // 32) * 36, dtype=torch.uint8, device=dev)
            qmv.quantize_q8_1(torch.from_numpy(x).to(dev), xq, DM, T)
            sets.append((torch.from_numpy(ids).to(dev), torch.from_numpy(rw).to(dev), xq,
                         len(set(ids.reshape(-1).tolist()))))
        wsb = qmv.grouped_expert_mmvq_workspace(E, T, TOPK, DM, DFF)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        o = torch.empty(T * DM, dtype=torch.float32, device=dev)

        def fn(sidx):
            ids, rw, xq, _ = sets[sidx]
            qmv.grouped_expert_mmvq(gd, ud, dp, qmv.LAYOUT_PLANAR, xq, ids, rw, o, E, T, TOPK, DM, DFF, ws, wsb)

        us = graph_avg_us(torch, [lambda i=i: fn(i) for i in range(len(sets))] * 4, reps=4)
        hit = sum(s[3] for s in sets) / len(sets)
        res[f"T{T}"] = {"avg_call_us": round(us, 3), "experts_hit_avg": hit,
                        "touched_weight_GBps": round(hit * per_expert / (us * 1e-6) / 1e9, 1)}
    return res


def cpu_baseline(np, synth, w_np, x_np, seconds):
    """The CPU oracle (plain scalar C, untuned) on the same step: quantize the
    13 columns, then the Q6_K product at N = 1, 4, 8 on their own columns.
    Timed twice: on one host core, and with the rows of each product split
    over all cores of the process's affinity mask (threads calling the
    oracle on row ranges; the oracle itself is unchanged).  The all-core
    figure is the reported value."""
    import concurrent.futures as cf
    import oracle as orc

    cores = max(1, min(len(os.sched_getaffinity(0)), 64))

    def one_step(pool, nthreads):
        xq = orc.quantize_q8_1(x_np)
        for n in NCOLS:
            xs = xq[COL0[n]:COL0[n] + n]
            if pool is None:
                orc.mmvq("q6k", w_np, xs, ROWS, K)
            else:
                per = (ROWS + nthreads - 1) // nthreads
                futs = [pool.submit(orc.mmvq, "q6k", w_np, xs, ROWS, K, r0, min(per, ROWS - r0))
                        for r0 in range(0, ROWS, per)]
                for f in futs:
                    f.result()

    def timed(pool, nthreads, budget):
        reps, t_total = 0, 0.0
        while t_total < budget or reps == 0:
            t0 = time.perf_counter()
            one_step(pool, nthreads)
            t_total += time.perf_counter() - t0
            reps += 1
        return t_total / reps, reps

    one_s, one_reps = timed(None, 1, seconds * 0.4)
    with cf.ThreadPoolExecutor(cores) as pool:
        all_s, all_reps = timed(pool, cores, seconds * 0.6)
    step_bytes = weight_bytes(ROWS, K) * len(NCOLS)
    return {"value": round(step_bytes / all_s / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"the full step (10240x2560 Q6_K, quantize 13 columns + products at N=1,4,8): "
                      f"{all_reps} steps at {all_s * 1e3:.1f} ms/step with rows split over {cores} threads; "
                      f"{one_reps} steps at {one_s * 1e3:.1f} ms/step "
                      f"({step_bytes / one_s / 1e9:.4f} GB/s) on one core",
            "ms_per_step": round(all_s * 1e3, 2),
            "one_core": {"value": round(step_bytes / one_s / 1e9, 4), "ms_per_step": round(one_s * 1e3, 2)}}


if __name__ == "__main__":
    main()
