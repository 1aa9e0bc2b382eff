#!/usr/bin/env python3
"""Benchmark of the DualScale x SegLinear W8A8 layer on one MI355X.

    python bench.py [--workload NAME] [--steps K] [--warmup W] [--gpus 1]

One step = one call of segquant_gemm_w8a8_seg: polarity split + dual-scale
quantisation of the bf16 activation, both int8 products against one weight
tile, per-segment fp32 rescale and bf16 store -- one kernel launch.  The
static scales and the packed weights are prepared before timing (offline in
the method).  Inputs are resident in HBM; R copies of them rotate so that no
cache (4 MB L2 per XCD, 256 MB MALL) holds a step's operands from the step
before.  The timed steps are replayed from a captured HIP graph (one graph of
R calls), bracketed by events and device synchronisation.

Prints ONE JSON line.  `value` is the workload's metric: GB/s of algorithmic
bytes (bf16 X + int8 W + bf16 Y) for the small-M AdaNorm layer (HBM bound),
effective TOPS (4*M*N*K int8 ops: both polarity halves) otherwise.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 matrix (5.0 POP/s)
METRIC = "DualScale seg-W8A8 GEMM effective TOPS & % int8 MFMA peak; GB/s at small M"
DEFAULT_WORKLOAD = "c2_adanorm_gemv"


def alg_bytes(wl) -> int:
    return 2 * wl.M * wl.K + wl.K * wl.N + 2 * wl.M * wl.N


def alg_ops(wl) -> int:
    return 4 * wl.M * wl.N * wl.K


def hbm_bound(wl) -> bool:
    # ridge of MI355X: 5.0e15 ops / 8.0e12 B/s = 625 ops per byte
    return alg_ops(wl) / alg_bytes(wl) < 625.0


def cpu_baseline(wl, x, w, seconds: float = 12.0):
    """The oracle, as it stands, on a bounded row sample of the workload."""
    import numpy as np
    import oracle
    nseg = None if wl.per_column else list(wl.nseg)
    sp, sn, ip, ineg = oracle.calibrate_amax(x, list(wl.kseg))
    wq, ws = oracle.quantize_weight(w, list(wl.kseg), nseg, wl.per_column)
    threads = oracle.num_threads()
    # rows per call: enough to give every thread rows, within ~seconds/3 per call
    macs_per_row = 2 * wl.K * wl.N
    rate_guess = 1.5e9 * threads  # int MACs/s, for sizing only
    rows = max(1, min(wl.M, int(rate_guess * seconds / 3 / macs_per_row)))
    rows = min(wl.M, max(rows, min(wl.M, threads)))
    xs = np.ascontiguousarray(x[:rows])
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        oracle.dualscale_linear(xs, wq, ws, list(wl.kseg), sp, sn, ip, ineg)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 50:
            break
    t = statistics.median(times)
    sub = wl.__class__(wl.name, wl.index, rows, wl.K, wl.N, wl.kseg, wl.nseg, wl.per_column)
    if hbm_bound(wl):
        value, unit = alg_bytes(sub) / t / 1e9, "GB/s"
    else:
        value, unit = alg_ops(sub) / t / 1e12, "TOPS"
    return {"value": value, "unit": unit, "cores": min(threads, rows), "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows (full K={wl.K}, N={wl.N}), median of {len(times)} "
                      f"calls of oracle_dualscale_linear (quantise, exact int32 products, fp64 "
                      f"dequantise); calibration and weight quantisation not timed",
            "seconds_per_call": t}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", default="bf16", choices=["bf16", "signed", "planes"],
                    help="bf16: fused quantisation (one launch); signed/planes: time the GEMM on "
                         "an activation pre-quantised by segquant_quantize_dualscale")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch each step from Python")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer is a single-GPU kernel library and this "
              "build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import segmented_dual_scale_amd as S
    from segmented_dual_scale_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    S.load_library()
    dev = torch.device("cuda:0")
    wl, x, w = W.make_inputs(args.workload)
    kseg = list(wl.kseg)
    nseg = None if wl.per_column else list(wl.nseg)

    # ---- offline: calibration + weight quantisation (not timed) ----
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    act = S.segquant_calibrate_amax(xd, kseg)
    wd = torch.from_numpy(w).to(dev)
    wp, ws = S.segquant_quantize_weight(wd, kseg, nseg, wl.per_column)
    del wd
    layout = {"signed": S.SEGQ_Q_SIGNED, "planes": S.SEGQ_Q_PLANES}.get(args.mode)
    xq = S.segquant_quantize_dualscale(xd, act, kseg, layout) if layout is not None else None
    torch.cuda.synchronize()

    # ---- rotating copies so no cache serves the operands ----
    set_bytes = alg_bytes(wl)
    R = max(1, min(64, math.ceil(640e6 / set_bytes)))
    xs = [xd] + [xd.clone() for _ in range(R - 1)]
    xqs = [xq] + [xq.clone() for _ in range(R - 1)] if xq is not None else [None] * R
    wps = [wp] + [wp.clone() for _ in range(R - 1)]
    ys = [torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    torch.cuda.synchronize()

    def step(i):
        j = i % R
        if xq is None:
            S.segquant_gemm_w8a8_seg(xs[j], wps[j], ws, act, kseg, out=ys[j])
        else:
            S.segquant_gemm_w8a8_seg(None, wps[j], ws, act, kseg, N=wl.N, xq=xqs[j],
                                     q_layout=layout, out=ys[j])

    stream = torch.cuda.Stream(device=dev)  # default priority
    use_graph = not args.no_graph
    with torch.cuda.stream(stream):
        for i in range(max(args.warmup, R)):
            step(i)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(R):
                step(i)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(max(1, args.warmup // R)):
                graph.replay()
        torch.cuda.synchronize()

    reps = max(1, math.ceil(args.steps / R)) if use_graph else 0
    steps = reps * R if use_graph else args.steps
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        if use_graph:
            for _ in range(reps):
                graph.replay()
        else:
            for i in range(steps):
                step(i)
        end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / steps

    if hbm_bound(wl):
        unit, value = "GB/s", alg_bytes(wl) / (ms_per_step * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": value, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": value / PEAK_HBM_GBS, "traffic": None}
    else:
        unit, value = "TOPS", alg_ops(wl) / (ms_per_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": value, "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": value / PEAK_INT8_TOPS, "traffic": None}
    kernel = "gemm_smallm_kernel" if S.segquant_gemm_kernel_for(wl.M, wl.N, wl.K) == \
        S.SEGQ_KERNEL_SMALLM else "gemm_tile_kernel"
    roof["kernel"] = kernel
    roof["per_launch"] = {"alg_bytes": alg_bytes(wl), "alg_int8_ops": alg_ops(wl),
                          "avg_us": ms_per_step * 1e3}

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded generators with the workload's shapes and polarity structure)",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N,
                   "k_segments": len(wl.kseg), "n_segments": len(wl.nseg),
                   "per_column_weight_scale": wl.per_column, "activation_input": args.mode,
                   "rotating_sets": R, "hip_graph": use_graph,
                   "useful_2mnk_tops": alg_ops(wl) / 2 / (ms_per_step * 1e-3) / 1e12},
        "roofline": roof,
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, x, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
