#!/usr/bin/env python3
"""Benchmark of the Q6_K MMVQ decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu] [--no-profile]

Workload (one "step"): quantize 13 fp32 activation columns to Q8_1 (the
column-planar arrangement of its bytes) in one launch, then the Q6_K MMVQ of
three 10240 x 2560 (rows x cols) matrices in the tiled layout (int8
matrix-core kernel) at N = 8, 4 and 1 columns -- each product on its own
weights and its own columns (8 + 4 + 1 = 13) -- issued as one batched launch
(mmvq_q6k_batch), as the decode products of a layer's matrices are.  This is
the decode matrix the pages measure as "2560 x 10240" (n_in x n_out) at 1-8
columns.  Weights are resident in HBM before timing and the step's three
products read three of 26 copies (559 MB, more than twice the 256 MB
Infinity Cache), rotating, so every weight byte comes from HBM.

Timing: exactly `steps` steps, replayed from HIP graphs holding
min(steps, 26) consecutive steps (and one graph for a remainder), between
two synchronizations; `value` = weight bytes of the three products / step
time (GB/s), the step time from HIP events on the launch stream around the
steps (the device's time, the wait for the first graph launch included;
the host wall time, which adds the host's own launch and synchronization
calls, is reported beside it).

`roofline` is for the dominant kernel (the batched launch): algorithmic
bytes per launch over its average launch duration, from HIP events on its
stream around graph replays of back-to-back launches (3 repeats of at least
2000 launches).  Before the GPU is touched, bench.py runs two short child
processes under rocprofv3: one with the FETCH_SIZE and one with the
WRITE_SIZE counter (HBM traffic per dispatch, scaled by what the same
counters read for a device copy of known size), and one kernel trace (per
kernel median, p10 and p90 dispatch durations, in three repeats); their
results go into the line (`roofline.traffic`, `extras.rocprof`).
`cpu_baseline` times the CPU oracle on the same step.  `extras` holds the
single launches per column count, the other shapes, the grouped MoE, a
cache-warm figure (not HBM) and calibration reads.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import math
import os
import shutil
import subprocess
import sys
import tempfile
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROWS, K = 10240, 2560
JOBS = (8, 4, 1)            # column counts of the step's three products, in launch order
NCOLS = (1, 4, 8)
XCOLS = sum(JOBS)           # distinct activation columns quantized per step
COL0 = {8: 0, 4: 8, 1: 12}  # first activation column of each product
Q6K_BYTES = 210
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2**20
BATCH_KERNEL = "k_mmvq_q6_tiled_jobs_stream<4, 4, 5, 4>"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
MOE_ROUTINGS = 32          # grouped MoE: routings replayed in turn per token count
SPIN_CYCLES = 1_000_000     # the untimed spin before the timed steps (shader clock: ~0.4 ms)
# pages' figures for this matrix (Arc A770, large-GRF launch, 1/4/8 columns):
# 86.1, 92.9, 370.5 us per call
PAGES_US = {1: 86.1, 4: 92.9, 8: 370.5}


def weight_bytes(rows, k, per_block=Q6K_BYTES):
    return rows * (k // 256) * per_block


def alg_bytes(rows, k, n, per_block=Q6K_BYTES):
    """Algorithmic bytes of one MMVQ: weights once, Q8_1 activations, fp32
    outputs."""
    return weight_bytes(rows, k, per_block) + n * (k // 32) * 36 + 4 * n * rows


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-profile", action="store_true",
                   help="skip the rocprofv3 child runs (traffic and kernel-trace statistics)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--pmc-workload", action="store_true",
                   help="only run 30 batched launches, 30 single launches per column count and 30 device copies "
                        "of the same 21.5 MB (the workload of the rocprofv3 --pmc passes), print nothing")
    p.add_argument("--trace-workload", action="store_true",
                   help="only run 3 repeats of at least 2000 batched launches and of single launches per column "
                        "count (the workload of the kernel trace), print nothing")
    p.add_argument("--pmc-dense", metavar="KIND:ROWSxK",
                   help="only run 30 launches each at 1 and 4 columns of the Q4_K or Q5_K product (e.g. "
                        "q4k:12288x2560) on rotated copies, 30 plain streaming reads of the same bytes and 30 "
                        "device copies of them (for rocprofv3 --pmc passes), print nothing")
    p.add_argument("--pmc-mmq", action="store_true",
                   help="only run 8 launches of the 512-column product mmq_q6k on the same matrix "
                        "(for rocprofv3 --pmc passes), print nothing")
    return p.parse_args()


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


def repeated_avg_us(torch, fn, nrot, min_launches=2000, repeats=3):
    """Per-launch device time (us) of fn(i), i = launch index: a graph of
    2*nrot back-to-back launches replayed until at least min_launches ran,
    events on the launch stream; `repeats` such measurements."""
    stream = torch.cuda.current_stream()
    per = 2 * nrot
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph, stream=stream):
        for i in range(per):
            fn(i)
    gph.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(min_launches / per))
    res = []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            gph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) * 1e3 / (reps * per))
    del gph
    return {"avg_launch_us": round(sum(res) / len(res), 3), "repeats_us": [round(v, 3) for v in res],
            "launches_per_repeat": reps * per}


# ----------------------------------------------------------- rocprofv3 runs
def _child(cmd, outdir, seconds):
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=HERE + os.pathsep + os.environ.get("PYTHONPATH", ""))
    try:
        r = subprocess.run(["timeout", "-s", "KILL", str(seconds), *cmd], cwd="/tmp", env=env,
                           capture_output=True, text=True)
    except OSError as e:
        return f"could not run rocprofv3: {e}"
    found = glob.glob(os.path.join(outdir, "**", "*.csv"), recursive=True)
    if r.returncode != 0 and not found:
        return f"rocprofv3 exit {r.returncode}: {(r.stderr or r.stdout)[-300:]}"
    return None


def _rows(outdir, suffix):
    rows = []
    for f in glob.glob(os.path.join(outdir, "**", f"*{suffix}"), recursive=True):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    n = name.split("(")[0].replace("void ", "").replace("qmv::", "")
    return n.strip()


def profile_children(py):
    """Traffic (two --pmc passes) and kernel-trace statistics of this
    script's own workloads, run under rocprofv3 as child processes before
    this process touches the GPU."""
    if shutil.which("rocprofv3") is None:
        return {"error": "rocprofv3 not found"}, None
    out = {}
    tmp = tempfile.mkdtemp(prefix="qmv_bench_prof_", dir="/tmp")
    try:
        # HBM traffic per dispatch, calibrated by a device copy of known size
        counters = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            d = os.path.join(tmp, c)
            err = _child(["rocprofv3", "--pmc", c, "--output-format", "csv", "-d", d, "-o", "pmc", "--",
                          py, "-u", os.path.join(HERE, "bench.py"), "--pmc-workload"], d, 120)
            if err:
                out["traffic_error"] = err
                break
            for r in _rows(d, "counter_collection.csv"):
                if r.get("Counter_Name") != c:
                    continue
                k = _short(r["Kernel_Name"])
                counters.setdefault(k, {}).setdefault(c, []).append(float(r["Counter_Value"]))
        if "traffic_error" not in out:
            copy = counters.get(COPY_KERNEL, {})
            wb = weight_bytes(ROWS, K)
            if not copy.get("FETCH_SIZE") or not copy.get("WRITE_SIZE"):
                out["traffic_error"] = "no copy-kernel counters for calibration"
            else:
                fk = sum(copy["FETCH_SIZE"]) / len(copy["FETCH_SIZE"])
                wk = sum(copy["WRITE_SIZE"]) / len(copy["WRITE_SIZE"])
                sf, sw = wb / (fk * 1024), wb / (wk * 1024)
                tr = {}
                for k, v in counters.items():
                    if "FETCH_SIZE" in v and "WRITE_SIZE" in v and k != COPY_KERNEL:
                        f = sum(v["FETCH_SIZE"]) / len(v["FETCH_SIZE"])
                        w = sum(v["WRITE_SIZE"]) / len(v["WRITE_SIZE"])
                        tr[k] = {"FETCH_SIZE_KiB": round(f, 1), "WRITE_SIZE_KiB": round(w, 1),
                                 "bytes": round(f * 1024 * sf + w * 1024 * sw), "dispatches": len(v["FETCH_SIZE"])}
                out["traffic"] = {"per_kernel": tr,
                                  "calibration": {"copy_bytes": wb, "FETCH_SIZE_KiB": round(fk, 1),
                                                  "WRITE_SIZE_KiB": round(wk, 1), "fetch_scale": round(sf, 4),
                                                  "write_scale": round(sw, 4)}}
        # kernel trace: per-kernel median / p10 / p90 in three repeats
        d = os.path.join(tmp, "trace")
        err = _child(["rocprofv3", "--kernel-trace", "--output-format", "csv", "-d", d, "-o", "tr", "--",
                      py, "-u", os.path.join(HERE, "bench.py"), "--trace-workload"], d, 180)
        if err:
            out["trace_error"] = err
        else:
            per = {}
            for r in _rows(d, "kernel_trace.csv"):
                per.setdefault(_short(r["Kernel_Name"]), []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            stats = {}
            for k, v in per.items():
                if "tiled" not in k or len(v) < 300:
                    continue
                v.sort()
                dur = [x[1] / 1e3 for x in v]
                third = len(dur) // 3
                reps = []
                for i in range(3):
                    s = sorted(dur[i * third:(i + 1) * third])
                    reps.append({"median_us": round(s[len(s) // 2], 3), "p10_us": round(s[len(s) // 10], 3),
                                 "p90_us": round(s[(9 * len(s)) // 10], 3), "dispatches": len(s)})
                a = sorted(dur)
                stats[k] = {"median_us": round(a[len(a) // 2], 3), "p10_us": round(a[len(a) // 10], 3),
                            "p90_us": round(a[(9 * len(a)) // 10], 3), "mean_us": round(sum(a) / len(a), 3),
                            "dispatches": len(a), "repeats": reps}
            out["kernel_trace"] = stats
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out, out.get("traffic")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this benchmark runs on one GPU only (the MMVQ would shard by output rows "
              "across GPUs; no multi-GPU path is built). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    workload_only = args.pmc_workload or args.trace_workload or args.pmc_mmq or args.pmc_dense
    prof, traffic = ({}, None)
    if not workload_only and not args.no_profile:
        prof, traffic = profile_children(sys.executable)

    import numpy as np
    import torch

    from quant_mat_vec_amd import qmv, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    # all work on one non-default stream (graph capture needs one; default
    # priority, like every stream here)
    torch.cuda.set_stream(torch.cuda.Stream())
    stream = torch.cuda.current_stream()
    if args.pmc_dense:
        dense_pmc_workload(torch, qmv, synth, dev, args.pmc_dense)
        return
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
    del w_gguf
    copies = [base.clone() for _ in range(ncopies)]
    xd = torch.from_numpy(x_np).to(dev)
    xq_all = torch.empty(XCOLS * (K // 32) * 36, dtype=torch.uint8, device=dev)
    qcol = (K // 32) * 36      # bytes of one Q8_1 column
    outs = {n: torch.empty(n * ROWS, dtype=torch.float32, device=dev) for n in JOBS}

    def xq_of(n):
        return xq_all[COL0[n] * qcol:(COL0[n] + n) * qcol]
    qmv.quantize_q8_1_planar(xd, xq_all, K, XCOLS)
    torch.cuda.synchronize()

    def batch(i):
        """The step's three products, on weight copies 3i, 3i+1, 3i+2."""
        qmv.mmvq_q6k_batch([(copies[(len(JOBS) * i + j) % ncopies], xq_of(n), outs[n], ROWS, n)
                            for j, n in enumerate(JOBS)], XT, K)

    def single(n):
        return lambda i: qmv.mmvq_q6k(copies[i % ncopies], XT, xq_of(n), outs[n], ROWS, K, n)

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
        # hardware-counter passes: the batched launch and the single products
        # on rotated copies, then a plain copy of the same size (its
        # FETCH_SIZE / WRITE_SIZE calibrate the counters against known bytes)
        for i in range(30):
            batch(i)
        for n in NCOLS:
            for i in range(30):
                single(n)(i)
        dst = torch.empty_like(base)
        for i in range(30):
            dst.copy_(copies[i % ncopies])
        torch.cuda.synchronize()
        return

    if args.trace_workload:
        # per kernel three consecutive repeats of at least 2000 launches (the
        # trace's thirds)
        repeated_avg_us(torch, batch, ncopies, min_launches=2000, repeats=3)
        for n in NCOLS:
            repeated_avg_us(torch, single(n), ncopies, min_launches=2000, repeats=3)
        return

    def step(i):
        qmv.quantize_q8_1_planar(xd, xq_all, K, XCOLS)
        batch(i)

    # Exactly `steps` steps: graphs of G = min(steps, ncopies) consecutive
    # steps (step offsets 0 .. G-1; with G = ncopies the rotation continues
    # across replays) and one graph for the remainder.
    graphs = {}

    def graph_of(n):
        if n not in graphs:
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph, stream=stream):
                for i in range(n):
                    step(i)
            graphs[n] = gph
        return graphs[n]

    def run_steps(n):
        G = min(n, ncopies)
        full, rest = divmod(n, G)
        for _ in range(full):
            graph_of(G).replay()
        if rest:
            graph_of(rest).replay()

    def timed_steps(n):
        run_steps(n)                       # capture and load every graph this count uses
        torch.cuda.synchronize()
        # device time of the n steps: a bounded spin kernel queued first keeps
        # the stream busy while the host enqueues the start event and the
        # graphs, so the events bracket the steps and not the host's
        # submission latency (one graph launch, ~5 % of 20 steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record(stream)
        run_steps(n)
        e1.record(stream)
        torch.cuda.synchronize()
        # host wall time of the same n steps from an idle stream
        t0 = time.perf_counter()
        run_steps(n)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return e0.elapsed_time(e1) / n, (t1 - t0) * 1e3 / n

    if args.warmup:
        run_steps(args.warmup)
        torch.cuda.synchronize()
    ms_per_step, wall_ms_per_step = timed_steps(args.steps)
    step_bytes = wb * len(JOBS)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # Per-launch averages: the batched launch (the dominant kernel) and the
    # single products per column count.
    qmv.quantize_q8_1_planar(xd, xq_all, K, XCOLS)
    bt = repeated_avg_us(torch, batch, ncopies)
    batch_alg = sum(alg_bytes(ROWS, K, n) for n in JOBS)
    per_n = {}
    for n in NCOLS:
        r = repeated_avg_us(torch, single(n), ncopies)
        per_n[str(n)] = dict(r, kernel=f"k_mmvq_q6_tiled<{n}, 4, 1, 5, false, false, true>",
                             weight_GBps=round(wb / (r["avg_launch_us"] * 1e-6) / 1e9, 1),
                             weight_frac_of_8TBps=round(wb / (r["avg_launch_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             alg_bytes=alg_bytes(ROWS, K, n))
    ach = batch_alg / (bt["avg_launch_us"] * 1e-6) / 1e9
    tr_bytes = None
    if traffic and BATCH_KERNEL in traffic.get("per_kernel", {}):
        tr_bytes = traffic["per_kernel"][BATCH_KERNEL]["bytes"]
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr_bytes,
                "kernel": BATCH_KERNEL, "jobs": "10240x2560 at 8, 4 and 1 columns",
                "alg_bytes_per_launch": batch_alg, "avg_launch_us": bt["avg_launch_us"],
                "launch_repeats_us": bt["repeats_us"], "launches_per_repeat": bt["launches_per_repeat"]}

    # checksum of the last N=8 output bits (FNV-1a 32)
    torch.cuda.synchronize()
    ob = outs[8].cpu().numpy().view(np.uint8)[:4096 * 4]
    h = np.uint32(2166136261)
    for byte in ob:
        h = np.uint32((int(h) ^ int(byte)) * 16777619 & 0xFFFFFFFF)

    extras = {"single_launch_per_ncols": per_n,
              "batched_launch": dict(bt, alg_bytes=batch_alg,
                                     weight_GBps=round(step_bytes / (bt["avg_launch_us"] * 1e-6) / 1e9, 1)),
              "wall_ms_per_step": round(wall_ms_per_step, 4),
              "steps_per_graph": min(args.steps, ncopies),
              "wall_clock_weight_GBps": round(step_bytes / (wall_ms_per_step * 1e-3) / 1e9, 1),
              "weight_copies": ncopies, "weight_bytes_per_copy": wb,
              "fnv1a32_out_prefix": int(h),
              "pages_A770_us": PAGES_US}
    if prof:
        extras["rocprof"] = prof
    if not args.no_extras:
        xq8 = xq_all[:8 * qcol]
        extras.update(run_extras(torch, np, qmv, synth, dev, copies, base, xd, xq8, outs[8]))

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
        "config": {"workload": "Q6_K MMVQ 10240x2560 (rows x cols), tiled weights (matrix cores), 8, 4 and 1 "
                               "columns on three weight copies in one batched launch, after one Q8_1 quantize "
                               "(column-planar layout) of the 13 activation columns; weights rotated over "
                               f"{ncopies} HBM copies",
                   "rows": ROWS, "cols": K, "ncols": list(JOBS),
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
        ex[f"{kind}_batch_12288_6144_512x2560"] = q45_batch_case(torch, qmv, synth, dev, kind)
    ex["moe_e128_2560_768"] = moe_case(torch, np, qmv, synth, dev)
    ex["rmsnorm_quantize_13x2560"] = norm_case(torch, np, qmv, synth, dev)
    ex["q6k_many_columns_mmq"] = {f"{r_}x{k_}": prefill_case(torch, qmv, synth, dev, r_, k_)
                                  for (r_, k_) in ((10240, 2560), (2560, 10240))}
    return ex


def q45_batch_case(torch, qmv, synth, dev, kind, k=2560, shapes=(12288, 6144, 512), ncols_list=(1, 4)):
    """The dense matrices of one K (12288, 6144 and 512 rows x 2560), each on
    its own weights, issued as one batch call (mmvq_q4k_batch /
    mmvq_q5k_batch: one launch, the 512-row matrix at twice the lanes per
    row of the others, as alone) and as three single calls; sets of weights
    rotated over HBM copies.  Per step:
    device time, weight GB/s, and the plain streaming read of the same
    bytes in one launch."""
    per = {"q4k": 144, "q5k": 176}[kind]
    g = synth.rng(31 + per)
    ws = [torch.from_numpy(synth.blocks(kind, g, r, k)).to(dev) for r in shapes]
    sbytes = sum(weight_bytes(r, k, per) for r in shapes)
    nc = max(2, math.ceil(2 * MALL_BYTES / sbytes) + 1)
    sets = [ws] + [[w.clone() for w in ws] for _ in range(nc - 1)]
    x = torch.from_numpy(synth.activations(g, max(ncols_list), k)).to(dev)
    q = torch.empty(max(ncols_list) * (k // 32) * 36, dtype=torch.uint8, device=dev)
    outs = [torch.empty(max(ncols_list) * r, dtype=torch.float32, device=dev) for r in shapes]
    bfn = qmv.mmvq_q4k_batch if kind == "q4k" else qmv.mmvq_q5k_batch
    sfn = qmv.mmvq_q4k if kind == "q4k" else qmv.mmvq_q5k
    res = {"weight_bytes_per_step": sbytes}
    for n in ncols_list:
        qmv.quantize_q8_1(x, q, k, n)
        jobs = [[(w, q, o, r, n) for w, o, r in zip(st, outs, shapes)] for st in sets]
        calls = [lambda jb=jb: bfn(jb, k) for jb in jobs] * max(1, 40 // len(jobs))
        bus = graph_avg_us(torch, calls, reps=4)
        calls = [lambda jb=jb: [sfn(w, q_, o, r, k, n_) for w, q_, o, r, n_ in jb] for jb in jobs]
        calls = calls * max(1, 40 // len(jobs))
        sus = graph_avg_us(torch, calls, reps=4)
        res[str(n)] = {"batch_us": round(bus, 3), "batch_weight_GBps": round(sbytes / (bus * 1e-6) / 1e9, 1),
                       "three_singles_us": round(sus, 3),
                       "three_singles_weight_GBps": round(sbytes / (sus * 1e-6) / 1e9, 1)}
    big = [torch.cat([w.view(-1) for w in st]) for st in sets[:nc]]
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    rb = sbytes // 4096 * 4096
    us = graph_avg_us(torch, [lambda c=c: qmv.qmv_stream_read(c, rb, sink, 0) for c in big] * 2)
    res["stream_read_same_bytes"] = {"avg_launch_us": round(us, 3), "read_GBps": round(rb / (us * 1e-6) / 1e9, 1)}
    del sets, big
    torch.cuda.empty_cache()
    return res


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


def dense_pmc_workload(torch, qmv, synth, dev, spec):
    """Counter workload of one Q4_K/Q5_K product: 30 launches at N = 1, then
    at N = 4, on weight copies rotated past the Infinity Cache; 30 plain
    streaming reads and 30 device copies of the same bytes."""
    kind, shape = spec.split(":")
    rows, k = (int(v) for v in shape.split("x"))
    g = synth.rng(synth.seed_for(3, 0, 0))
    blk = synth.q4k_blocks(g, rows, k) if kind == "q4k" else synth.q5k_blocks(g, rows, k)
    base = torch.from_numpy(blk).to(dev)
    copies = [base.clone() for _ in range(max(2, math.ceil(2 * MALL_BYTES / blk.size) + 1))]
    fn = qmv.mmvq_q4k if kind == "q4k" else qmv.mmvq_q5k
    for n in (1, 4):
        xq = torch.empty(n * (k // 32) * 36, dtype=torch.uint8, device=dev)
        qmv.quantize_q8_1(torch.from_numpy(synth.activations(g, n, k)).to(dev), xq, k, n)
        out = torch.empty(n * rows, dtype=torch.float32, device=dev)
        for i in range(30):
            fn(copies[i % len(copies)], xq, out, rows, k, n)
    sink = torch.empty(1 << 18, dtype=torch.int32, device=dev)
    for i in range(30):
        qmv.qmv_stream_read(copies[i % len(copies)], blk.size // 16 * 16, sink, 0)
    dst = torch.empty_like(base)
    for i in range(30):
        dst.copy_(copies[i % len(copies)])
    torch.cuda.synchronize()


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
        # different routings, replayed in turn: 32 of them touch 112-128 of
        # the experts (409-467 MiB), so that the cycle does not fit the
        # 256 MiB Infinity Cache and expert weights come from HBM (eight
        # routings of one token touch ~55 experts, ~200 MiB, and measured
        # 12.4 against 13.4 us per call)
        sets = []
        for s in range(MOE_ROUTINGS):
            ids, rw = synth.routing(synth.rng(1000 + 100 * T + s), T, E, TOPK)
            x = synth.activations(synth.rng(2000 + 100 * T + s), T, DM)
            xq = torch.empty(T * (DM // 32) * 36, dtype=torch.uint8, device=dev)
            qmv.quantize_q8_1(torch.from_numpy(x).to(dev), xq, DM, T)
            sets.append((torch.from_numpy(ids).to(dev), torch.from_numpy(rw).to(dev), xq,
                         len(set(ids.reshape(-1).tolist())), set(ids.reshape(-1).tolist())))
        wsb = qmv.grouped_expert_mmvq_workspace(E, T, TOPK, DM, DFF)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        o = torch.empty(T * DM, dtype=torch.float32, device=dev)

        def fn(sidx):
            ids, rw, xq = sets[sidx][:3]
            qmv.grouped_expert_mmvq(gd, ud, dp, qmv.LAYOUT_PLANAR, xq, ids, rw, o, E, T, TOPK, DM, DFF, ws, wsb)

        us = graph_avg_us(torch, [lambda i=i: fn(i) for i in range(len(sets))], reps=4)
        hit = sum(s[3] for s in sets) / len(sets)
        cycle = len(set().union(*(s[4] for s in sets)))
        res[f"T{T}"] = {"avg_call_us": round(us, 3), "experts_hit_avg": hit,
                        "experts_in_cycle": cycle, "routings": len(sets),
                        "touched_weight_GBps": round(hit * per_expert / (us * 1e-6) / 1e9, 1),
                        "frac_of_8TBps": round(hit * per_expert / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
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
            "cpu_model": cpu_model(),
            "sample": f"the full step (10240x2560 Q6_K, quantize 13 columns + products at N=1,4,8): "
                      f"{all_reps} steps at {all_s * 1e3:.1f} ms/step with rows split over {cores} threads; "
                      f"{one_reps} steps at {one_s * 1e3:.1f} ms/step "
                      f"({step_bytes / one_s / 1e9:.4f} GB/s) on one core",
            "ms_per_step": round(all_s * 1e3, 2),
            "one_core": {"value": round(step_bytes / one_s / 1e9, 4), "ms_per_step": round(one_s * 1e3, 2)}}


if __name__ == "__main__":
    main()
