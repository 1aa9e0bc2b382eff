#!/usr/bin/env python3
"""Benchmark of the DualScale x SegLinear W8A8 layer on one MI355X.

    python bench.py [--workload NAME] [--steps K] [--warmup W] [--gpus 1]

One step = one call of segquant_gemm_w8a8_seg: polarity split + dual-scale
quantisation of the bf16 activation, both int8 products against one weight
tile, per-segment fp32 rescale and bf16 store.  That is one kernel launch,
or two (quantisation into a workspace, then the GEMM from the codes) for the
wide layers where the library asks for a workspace; the roofline is then the
GEMM kernel's, timed on its own.  The
static scales and the packed weights are prepared before timing (offline in
the method).  Inputs are resident in HBM; R copies of them rotate so that no
cache (4 MB L2 per XCD, 256 MB MALL) holds a step's operands from the step
before.  The timed steps are replayed from a captured HIP graph (one graph of
R calls) on a stream of our own, bracketed by HIP events on that stream and
device synchronisation.

Prints ONE JSON line.  `value` is the workload's metric: GB/s of algorithmic
bytes (bf16 X + int8 W + bf16 Y) for the small-M AdaNorm layer (HBM bound),
effective TOPS (4*M*N*K int8 ops: both polarity halves) otherwise.  The line
also carries the roofline of the kernel (with the HBM traffic measured by
rocprofv3 counters when a counter record of the current kernel source exists
under profiles/), the CPU oracle timed on a bounded sample, and the same
measurement for every named workload ("all_workloads").

Counter passes (run under rocprofv3 --pmc, one counter per run):
    python bench.py --workload NAME --pmc-pass
runs a few plain (non-graph) steps and then a copy of known size (the scale
of the byte counters).  --ingest-pmc FETCH_DIR WRITE_DIR turns the two runs'
CSV output into the counter record profiles/traffic_<kernel>_<workload>.txt.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
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
COPY_PROBE_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "segmented_dual_scale_amd", "csrc")
KERNEL_SOURCES = {
    "gemm_smallm_kernel": ["gemm_smallm.hip", "sq_device.hpp", "sq_launch.hpp"],
    "gemm_tile_kernel": ["gemm_tile.hip", "sq_device.hpp", "sq_launch.hpp"],
    "gemm_lds_kernel": ["gemm_lds.hip", "sq_device.hpp", "sq_launch.hpp"],
}
RUNNING_SUM_MAX_K = 132104  # K * 128 * 127 < 2^31: the tile kernel's running int32 sums
# The pages' own timing figures: whole-model, per denoising step, not per layer.
PAGES_LATENCY = ("hliangzhao.me 'SegQuant' page, deployment-cost table (SD3.5 on an RTX 4090, "
                 "whole backbone per sampling step): FP16 317.18 ms, INT8 baseline 278.86 ms, "
                 "SegQuant-8 287.85 ms, INT4 baseline 209.78 ms, SegQuant-4 212.87 ms; the "
                 "pages give no per-layer or per-kernel latency")


def alg_bytes(wl) -> int:
    return 2 * wl.M * wl.K + wl.K * wl.N + 2 * wl.M * wl.N


def alg_ops(wl) -> int:
    return 4 * wl.M * wl.N * wl.K


def hbm_bound(wl) -> bool:
    # ridge of MI355X: 5.0e15 ops / 8.0e12 B/s = 625 ops per byte
    return alg_ops(wl) / alg_bytes(wl) < 625.0


def gemm_kernel_name(M: int, K: int, kseg, codes: bool, smallm: bool) -> str:
    """The kernel that runs the GEMM launch of a call: the streaming small-M
    kernel; the LDS-staged kernel for several K-segments on int8 codes (or K
    beyond the running-sum bound); otherwise the tile kernel (one segment, or
    every segment one 64-wide step)."""
    if smallm:
        return "gemm_smallm_kernel"
    widths = list(kseg)
    if len(widths) > 1 and any(w != 64 for w in widths) and (codes or K > RUNNING_SUM_MAX_K):
        return "gemm_lds_kernel"
    return "gemm_tile_kernel"


def workload_kernel(S, wl, mode: str) -> str:
    """gemm_kernel_name for a workload run in one of the bench's modes."""
    flags = {"single": S.SEGQ_GEMM_SINGLE_SCALE, "w4": S.SEGQ_GEMM_W4}.get(mode, S.SEGQ_GEMM_AUTO)
    kseg = list(wl.kseg)
    smallm = S.segquant_gemm_kernel_for(wl.M, wl.N, wl.K, flags) == S.SEGQ_KERNEL_SMALLM
    # the workspace holds the int8 widening of 4-bit weights (K*N, off the
    # small-M path) and, when the call quantises first, the M*K codes
    widen = wl.K * wl.N if mode == "w4" and not smallm else 0
    codes = mode in ("signed", "planes") or \
        S.segquant_gemm_workspace_bytes(wl.M, wl.N, wl.K, kseg, flags) - widen >= wl.M * wl.K
    return gemm_kernel_name(wl.M, wl.K, kseg, codes, smallm)


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")


def read_traffic(kernel: str, workload: str, mode: str):
    """HBM bytes per launch from the counter record, or None when there is no
    record for this kernel source (the kernel changed since it was taken)."""
    path = traffic_record_path(kernel, workload)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != source_digest(kernel) or rec.get("mode") != mode:
        return None
    fetch_f = float(rec["copy_fetch_kib"]) * 1024 / float(rec["copy_bytes"])
    write_f = float(rec["copy_write_kib"]) * 1024 / float(rec["copy_bytes"])
    fetch = float(rec["fetch_kib_per_dispatch"]) * 1024 / fetch_f
    write = float(rec["write_kib_per_dispatch"]) * 1024 / write_f
    return {"bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
            "copy_scale_fetch": fetch_f, "copy_scale_write": write_f,
            "record": os.path.relpath(path, ROOT)}


def trace_record_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"trace_{kernel}_{workload}.txt")


def read_trace(kernel: str, workload: str, mode: str):
    """Per-dispatch duration statistics of the kernel from the committed
    rocprofv3 kernel-trace record, or None when there is none for the current
    kernel source."""
    path = trace_record_path(kernel, workload)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != source_digest(kernel) or rec.get("mode") != mode:
        return None
    out = {k: float(rec[k]) for k in ("calls", "mean_us", "p10_us", "median_us", "p90_us")}
    out["calls"] = int(out["calls"])
    out["record"] = os.path.relpath(path, ROOT)
    return out


def _trace_spans(run_dir: str):
    """{kernel name: [(start, end) ns, in start order]} of a kernel-trace run."""
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {run_dir}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                per.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    for v in per.values():
        v.sort()
    return per


def _trace_durations(run_dir: str):
    return {k: [e - s for s, e in v] for k, v in _trace_spans(run_dir).items()}


def _stats_us(v):
    v = sorted(v)
    n = len(v)
    return {"calls": n, "mean_us": sum(v) / n / 1e3, "p10_us": v[n // 10] / 1e3,
            "median_us": v[n // 2] / 1e3, "p90_us": v[(9 * n) // 10] / 1e3}


def ingest_trace(run_dir: str, workload: str, mode: str, kernel: str, command: str,
                 timed: int):
    """Write the kernel-trace record of the layer kernel on one workload from
    a rocprofv3 --kernel-trace run of the headline phase alone.  The record's
    statistics cover the timed replay: the last `timed` dispatches of the
    kernel in start order (the benchmark replays its graph of `steps` calls
    once untimed, then once timed, after eager warm-up calls)."""
    spans = _trace_spans(run_dir)
    mine = sorted(sp for name, v in spans.items() if kernel in name for sp in v)
    if len(mine) < timed:
        raise SystemExit(f"{len(mine)} dispatches of {kernel} in {run_dir}, fewer than {timed}")
    last = mine[-timed:]
    st = _stats_us([e - s for s, e in last])
    gaps = [last[i + 1][0] - last[i][1] for i in range(len(last) - 1)]
    allst = _stats_us([e - s for s, e in mine])
    path = trace_record_path(kernel, workload)
    with open(path, "w") as fh:
        fh.write(f"# Dispatch durations (End - Start) of {kernel} on {workload} ({mode}\n"
                 f"# activation input), from a rocprofv3 kernel trace of the benchmark's\n"
                 f"# headline phase alone (no other workload, no single-scale launches):\n"
                 f"#   {command}\n"
                 f"# The statistics are those of the timed replay: the last {timed} dispatches\n"
                 f"# of the kernel.  The tracer inserts gaps between dispatches (mean\n"
                 f"# {sum(gaps) / max(1, len(gaps)) / 1e3:.2f} us here); the benchmark's own event\n"
                 f"# timing of the same replay without the tracer includes the real gaps.\n"
                 f"# All {allst['calls']} dispatches of the run (eager warm-up included): mean\n"
                 f"# {allst['mean_us']:.2f} us, median {allst['median_us']:.2f} us.\n"
                 f"# source_sha256 covers {', '.join(KERNEL_SOURCES[kernel])}.\n")
        fh.write(f"kernel: {kernel}\nworkload: {workload}\nmode: {mode}\n")
        fh.write(f"source_sha256: {source_digest(kernel)}\n")
        for k in ("calls", "mean_us", "p10_us", "median_us", "p90_us"):
            fh.write(f"{k}: {st[k]:.4f}\n" if k != "calls" else f"{k}: {st[k]}\n")
        fh.write("# every kernel of the run (all dispatches):\n")
        for name, v in sorted(spans.items(), key=lambda kv: -sum(e - s for s, e in kv[1])):
            s2 = _stats_us([e - s for s, e in v])
            fh.write(f"#   {s2['calls']:6d} calls  mean {s2['mean_us']:9.2f} us  median "
                     f"{s2['median_us']:9.2f} us  {name[:120]}\n")
    print(open(path).read())


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
        if time.perf_counter() > t_end or len(times) >= 10000:
            break
    t = statistics.median(times)
    sub = wl.__class__(wl.name, wl.index, rows, wl.K, wl.N, wl.kseg, wl.nseg, wl.per_column)
    if hbm_bound(wl):
        value, unit = alg_bytes(sub) / t / 1e9, "GB/s"
    else:
        value, unit = alg_ops(sub) / t / 1e12, "TOPS"
    used = min(threads, rows)  # the oracle parallelises over rows only
    host = len(os.sched_getaffinity(0))
    return {"value": value, "unit": unit, "cores": used, "threads_used": used,
            "host_cores": host, "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows (full K={wl.K}, N={wl.N}), median of {len(times)} "
                      f"calls of oracle_dualscale_linear (quantise, exact int32 products, fp64 "
                      f"dequantise) over {sum(times):.1f} s on {used} of the {host} host cores "
                      f"this process may use (OpenMP over rows: at most one thread per row); "
                      f"calibration and weight quantisation not timed",
            "seconds_per_call": t}


class Layer:
    """One workload's operands on the GPU, R rotating copies."""

    def __init__(self, S, W, dev, name: str, mode: str, rotate: bool = True):
        import numpy as np
        import torch
        self.S, self.mode = S, mode
        # single: the single-scale W8A8 baseline (one symmetric scale per
        # segment, one product), bf16 input
        self.flags = {"single": S.SEGQ_GEMM_SINGLE_SCALE, "w4": S.SEGQ_GEMM_W4}.get(
            mode, S.SEGQ_GEMM_AUTO)
        wl, x, w = W.make_inputs(name)
        self.wl, self.x, self.w = wl, x, w
        self.kseg = list(wl.kseg)
        nseg = None if wl.per_column else list(wl.nseg)
        # offline: calibration + weight quantisation (not timed)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.act = (S.segquant_calibrate_amax_single(xd, self.kseg) if mode == "single"
                    else S.segquant_calibrate_amax(xd, self.kseg))
        wd = torch.from_numpy(w).to(dev)
        wp, self.ws = S.segquant_quantize_weight(wd, self.kseg, nseg, wl.per_column,
                                                 bits=4 if mode == "w4" else 8)
        del wd
        self.layout = {"signed": S.SEGQ_Q_SIGNED, "planes": S.SEGQ_Q_PLANES}.get(mode)
        self.w_bytes = wl.K * wl.N // (2 if mode == "w4" else 1)
        xq = S.segquant_quantize_dualscale(xd, self.act, self.kseg, self.layout) \
            if self.layout is not None else None
        torch.cuda.synchronize()
        R = max(1, min(64, math.ceil(640e6 / self.alg_bytes()))) if rotate else 1
        self.R = R
        if xq is None:
            self.xs = [xd] + [xd.clone() for _ in range(R - 1)]
            self.xqs = [None] * R
        else:
            del xd
            self.xs = [None] * R
            self.xqs = [xq] + [xq.clone() for _ in range(R - 1)]
        self.wps = [wp] + [wp.clone() for _ in range(R - 1)]
        self.ys = [torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        torch.cuda.synchronize()
        self.kernel = workload_kernel(S, wl, mode)
        # the library's choice of quantising first (one workspace, reused by
        # every call, as a layer would)
        nb = S.segquant_gemm_workspace_bytes(wl.M, wl.N, wl.K, self.kseg, self.flags) \
            if self.layout is None else 0
        self.work = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        self.launches = 2 if nb else 1
        self.gemm_only = False  # time the GEMM launch alone, from the workspace codes

    def step(self, i: int):
        S, j = self.S, i % self.R
        if self.gemm_only:
            S.segquant_gemm_w8a8_seg(None, self.wps[j], self.ws, self.act, self.kseg,
                                     N=self.wl.N, xq=self.work.view(self.wl.M, self.wl.K),
                                     q_layout=S.SEGQ_Q_SIGNED, out=self.ys[j], flags=self.flags)
        elif self.layout is None:
            S.segquant_gemm_w8a8_seg(self.xs[j], self.wps[j], self.ws, self.act, self.kseg,
                                     out=self.ys[j], workspace=self.work, flags=self.flags)
        else:
            S.segquant_gemm_w8a8_seg(None, self.wps[j], self.ws, self.act, self.kseg,
                                     N=self.wl.N, xq=self.xqs[j], q_layout=self.layout,
                                     out=self.ys[j])

    def time(self, stream, steps: int, warmup: int, use_graph: bool, min_seconds: float = 0.0):
        """Average ms per step.  min_seconds == 0: exactly `steps` timed steps,
        one graph of `steps` calls over the rotating sets, replayed once
        untimed and then once timed.  min_seconds > 0 (the summary of all
        workloads): whole replays of a graph of one call per set, as many as
        fill min_seconds (and at least `steps` steps)."""
        import torch
        R = self.R
        with torch.cuda.stream(stream):
            for i in range(max(warmup, R)):
                self.step(i)
        torch.cuda.synchronize()
        if use_graph and min_seconds <= 0:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(steps):
                    self.step(i)
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                graph.replay()
            torch.cuda.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                start.record(stream)
                graph.replay()
                end.record(stream)
            torch.cuda.synchronize()
            del graph
            return start.elapsed_time(end) / steps, steps
        graph = None
        if use_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(R):
                    self.step(i)
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for _ in range(max(1, warmup // R)):
                    graph.replay()
            torch.cuda.synchronize()
            reps = max(1, math.ceil(steps / R))
            if min_seconds > 0:  # size the timed region from one timed replay
                t0 = time.perf_counter()
                with torch.cuda.stream(stream):
                    graph.replay()
                torch.cuda.synchronize()
                reps = max(reps, math.ceil(min_seconds / max(time.perf_counter() - t0, 1e-6)))
            n = reps * R
        else:
            n = steps
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            start.record(stream)
            if use_graph:
                for _ in range(n // R):
                    graph.replay()
            else:
                for i in range(n):
                    self.step(i)
            end.record(stream)
        torch.cuda.synchronize()
        del graph
        return start.elapsed_time(end) / n, n

    def alg_bytes(self) -> int:
        """bf16 X + weight (int8, or 4-bit) + bf16 Y."""
        wl = self.wl
        return 2 * wl.M * wl.K + self.w_bytes + 2 * wl.M * wl.N

    def metrics(self, ms_per_step: float):
        wl = self.wl
        if hbm_bound(wl):
            v = self.alg_bytes() / (ms_per_step * 1e-3) / 1e9
            return {"value": v, "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
                    "frac": v / PEAK_HBM_GBS}
        v = alg_ops(wl) / (ms_per_step * 1e-3) / 1e12
        return {"value": v, "unit": "TOPS", "bound": "mfma", "peak": PEAK_INT8_TOPS,
                "frac": v / PEAK_INT8_TOPS}

    def gemm_ms(self, stream, steps: int, warmup: int, use_graph: bool, min_seconds: float = 0.0):
        """ms per launch of the GEMM kernel alone (two-launch steps only)."""
        self.gemm_only = True
        try:
            return self.time(stream, steps, warmup, use_graph, min_seconds)[0]
        finally:
            self.gemm_only = False

    def free(self):
        self.xs = self.xqs = self.wps = self.ys = self.work = None


def measured_peaks(dev, stream, slab_bytes: int = 0, sustain_s: float = 1.0):
    """Ceilings measured on this GPU by the probe library: an int8
    matrix-core-only loop (one wave per SIMD and two), the shader clock while
    it runs, a streaming read and a device copy of 1 GiB, and (slab_bytes > 0)
    the time per launch of streaming slab_bytes from HBM, launches back to
    back in a graph over distinct slices of the 1 GiB buffer (so no slice is
    in a cache), best of several grid sizes."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "segmented_dual_scale_amd", "libsegquant_probe.so")
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.sqprobe_mfma_i8.argtypes = [I64, I32, I32, P, P, P]
    lib.sqprobe_stream_read.argtypes = [P, I64, I32, P, P]
    lib.sqprobe_ops_per_mfma.restype = I64
    lib.sqprobe_mfma_i8_data.argtypes = [I64, I32, I32, P, P, P, P]
    lib.sqprobe_mfma_data_bytes_per_wave.restype = I64
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sp = ctypes.c_void_p(stream.cuda_stream)
    khz = lib.sqprobe_wall_clock_khz()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return best

    out = {}
    iters = 40000
    best_tops, clock = 0.0, None
    for blocks_per_cu in (1, 2):
        blocks = cus * blocks_per_cu
        waves = blocks * 4
        sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
        spans = torch.zeros(waves * 2, dtype=torch.int64, device=dev)

        def run():
            rc = lib.sqprobe_mfma_i8(iters, blocks, 4, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(spans.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"sqprobe_mfma_i8 failed ({rc})")
        with torch.cuda.stream(stream):
            t = timed(run, 3)
        ops = waves * iters * lib.sqprobe_mfma_chains() * lib.sqprobe_ops_per_mfma()
        tops = ops / t / 1e12
        sv = spans.view(-1, 2).cpu().double()
        ratio = float((sv[:, 0] / sv[:, 1].clamp(min=1)).median())
        out[f"mfma_loop_{blocks_per_cu}wg_per_cu_tops"] = tops
        if tops > best_tops:
            best_tops = tops
            clock = ratio * khz * 1e3 if khz > 0 else None
    out["int8_mfma_tops"] = best_tops
    out["shader_clock_ghz_under_mfma"] = clock / 1e9 if clock else None
    # the same loop sustained: back-to-back launches for about `sustain_s`
    # seconds, rate and clock over the last ones (the clock falls under a
    # long matrix-core load; the layer kernels run that long in a serving loop)
    if sustain_s > 0:
        blocks = cus
        waves = blocks * 4
        sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
        spans = torch.zeros(waves * 2, dtype=torch.int64, device=dev)

        def run1():
            rc = lib.sqprobe_mfma_i8(iters, blocks, 4, ctypes.c_void_p(sink.data_ptr()),
                                     ctypes.c_void_p(spans.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"sqprobe_mfma_i8 failed ({rc})")
        with torch.cuda.stream(stream):
            t1 = timed(run1, 1)
            n = max(32, int(sustain_s / t1))
            last = 16
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for i in range(n):
                if i == n - last:
                    e0.record(stream)
                run1()
            e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / last
        ops = waves * iters * lib.sqprobe_mfma_chains() * lib.sqprobe_ops_per_mfma()
        sv = spans.view(-1, 2).cpu().double()
        ratio = float((sv[:, 0] / sv[:, 1].clamp(min=1)).median())
        out["mfma_loop_sustained_tops"] = ops / t / 1e12
        out["shader_clock_ghz_sustained_mfma"] = ratio * khz * 1e3 / 1e9 if khz > 0 else None
        out["mfma_loop_sustained_seconds"] = n * t
        # the same, sustained, on random operands that change every instruction
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        src = torch.randint(-128, 128, (waves * lib.sqprobe_mfma_data_bytes_per_wave(),),
                            dtype=torch.int8, device=dev, generator=gen)

        def run_data():
            rc = lib.sqprobe_mfma_i8_data(iters, blocks, 4, ctypes.c_void_p(src.data_ptr()),
                                          ctypes.c_void_p(sink.data_ptr()),
                                          ctypes.c_void_p(spans.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"sqprobe_mfma_i8_data failed ({rc})")
        with torch.cuda.stream(stream):
            t1 = timed(run_data, 1)
            n = max(32, int(sustain_s / t1))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for i in range(n):
                if i == n - last:
                    e0.record(stream)
                run_data()
            e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / last
        sv = spans.view(-1, 2).cpu().double()
        ratio = float((sv[:, 0] / sv[:, 1].clamp(min=1)).median())
        out["mfma_loop_data_tops"] = ops / t / 1e12
        out["shader_clock_ghz_data_mfma"] = ratio * khz * 1e3 / 1e9 if khz > 0 else None
        del src
    nbytes = 1 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    blocks = cus * 8
    rsink = torch.empty(16 * cus * 256, dtype=torch.int32, device=dev)  # also the slab probe's

    def read():
        rc = lib.sqprobe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks,
                                     ctypes.c_void_p(rsink.data_ptr()), sp)
        if rc != 0:
            raise RuntimeError(f"sqprobe_stream_read failed ({rc})")
    with torch.cuda.stream(stream):
        t = timed(read, 5)
    out["hbm_read_gbs"] = nbytes / t / 1e9
    if slab_bytes > 0:
        slab = (slab_bytes + 255) // 256 * 256
        nslab = nbytes // slab
        best_us, best_blocks = float("inf"), None
        for blocks in (cus // 2, cus, 2 * cus, 4 * cus, 8 * cus, 16 * cus):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(nslab):
                    rc = lib.sqprobe_stream_read(ctypes.c_void_p(buf.data_ptr() + i * slab), slab,
                                                 blocks, ctypes.c_void_p(rsink.data_ptr()), sp)
                    if rc != 0:
                        raise RuntimeError(f"sqprobe_stream_read failed ({rc})")
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(5):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (5 * nslab)
            if us < best_us:
                best_us, best_blocks = us, blocks
            del g
        out["hbm_stream_slab_bytes"] = slab
        out["hbm_stream_slab_us"] = best_us
        out["hbm_stream_slab_blocks"] = best_blocks
    half = nbytes // 2
    src, dst = buf[:half], buf[half:]
    with torch.cuda.stream(stream):
        t = timed(lambda: dst.copy_(src), 5)
    out["hbm_copy_gbs"] = 2 * half / t / 1e9
    out["method"] = (f"probe library: int8 32x32x32 matrix-core loop, {lib.sqprobe_mfma_chains()} "
                     f"independent accumulators per wave, 4 waves per workgroup, 1 and 2 "
                     f"workgroups per CU ({cus} CUs), clock = shader/constant clock ratio "
                     f"over the loop; the 1-per-CU loop again back to back for about "
                     f"{sustain_s:g} s, rate and clock over the last launches (sustained), and "
                     f"likewise on random operands that change every instruction (data); "
                     f"grid-stride 16-byte read of 1 GiB; torch copy of 512 MiB; "
                     f"best of 3-5 timed launches; slab: grid-stride reads of slab_bytes from "
                     f"{nbytes // max(slab_bytes, 1) if slab_bytes else 0} distinct slices, one launch "
                     f"each, replayed as a graph, best of {cus // 2}-{16 * cus} workgroups")
    del buf, rsink
    return out


def producer_fusion(S, W, dev, stream, names=("c2_adanorm_gemv", "c3_dit_ffn_fc2",
                                                 "c5_flux_ffn_fc2")):
    """The activation fused with the quantisation against the two passes it
    replaces (activation to bf16 X in HBM, then quantisation), on the
    pre-activations of the workloads whose X is SiLU/GELU output.  Codes as
    signed int8; rotating copies of Z so the caches do not hold a step's
    input."""
    import numpy as np
    import torch
    out = {}
    for name in names:
        wl = W.WORKLOADS[name]
        kind = W.preact_kind(wl)
        act_kind = S.SEGQ_ACT_SILU if kind == "silu" else S.SEGQ_ACT_GELU
        z0 = torch.from_numpy(W.make_preact(wl).view(np.int16)).to(dev).view(torch.bfloat16)
        kseg = list(wl.kseg)
        _, x = S.segquant_activate_quantize(z0, act_kind, kseg=kseg, x_out=True, want_codes=False)
        act = S.segquant_calibrate_amax(x, kseg)
        elems = wl.M * wl.K
        R = max(1, min(16, math.ceil(640e6 / (2 * elems))))
        zs = [z0] + [z0.clone() for _ in range(R - 1)]
        q = torch.empty((wl.M, wl.K), dtype=torch.int8, device=dev)

        def fused(i):
            S.segquant_activate_quantize(zs[i % R], act_kind, act, kseg, S.SEGQ_Q_SIGNED, out=q)

        def unfused(i):
            S.segquant_activate_quantize(zs[i % R], act_kind, kseg=kseg, x_out=x, want_codes=False)
            S.segquant_quantize_dualscale(x, act, kseg, S.SEGQ_Q_SIGNED, out=q)

        res = {}
        for label, fn in (("fused", fused), ("unfused", unfused)):
            with torch.cuda.stream(stream):
                for i in range(2 * R):
                    fn(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(R):
                    fn(i)
            reps = max(1, math.ceil(40 / R))
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            res[label + "_us"] = e0.elapsed_time(e1) * 1e3 / (reps * R)
            del g
        res["activation"] = kind
        res["elements"] = elems
        res["fused_gbs"] = 3 * elems / (res["fused_us"] * 1e-6) / 1e9   # 2 B read, 1 B written
        res["unfused_over_fused"] = res["unfused_us"] / res["fused_us"]
        out[name] = res
        del zs, x, q, z0
        torch.cuda.empty_cache()
    return out


def copy_probe(dev, reps: int = 3):
    """A copy of known size (the scale of the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    src = torch.randint(0, 1 << 30, (COPY_PROBE_BYTES // 4,), dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()


def _counter_means(run_dir: str, name_part: str):
    """Mean per dispatch of each counter over kernels whose name contains name_part."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if name_part not in r["Kernel_Name"]:
                    continue
                key = (f, r["Dispatch_Id"])
                d = per.setdefault(r["Counter_Name"], {})
                d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    return {c: (sum(d.values()) / len(d), len(d)) for c, d in per.items()}


def ingest_pmc(fetch_dir: str, write_dir: str, workload: str, mode: str, kernel: str,
               command: str):
    f_k = _counter_means(fetch_dir, kernel)["FETCH_SIZE"]
    w_k = _counter_means(write_dir, kernel)["WRITE_SIZE"]
    f_c = _counter_means(fetch_dir, "bitwise_not")["FETCH_SIZE"]
    w_c = _counter_means(write_dir, "bitwise_not")["WRITE_SIZE"]
    path = traffic_record_path(kernel, workload)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of {kernel} on {workload} ({mode} activation input), from\n"
                 f"# rocprofv3 counters, one counter per run (mean over dispatches):\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            fh.write(f"#   rocprofv3 --pmc {c} -d <dir> -o pmc --output-format csv -- {command}\n")
        fh.write(f"# The copy probe is torch.bitwise_not over {COPY_PROBE_BYTES} bytes of int32\n"
                 f"# (reads and writes that many bytes): its counters give the KiB scale.\n"
                 f"# source_sha256 covers {', '.join(KERNEL_SOURCES[kernel])}.\n")
        fh.write(f"kernel: {kernel}\nworkload: {workload}\nmode: {mode}\n")
        fh.write(f"source_sha256: {source_digest(kernel)}\n")
        fh.write(f"fetch_kib_per_dispatch: {f_k[0]:.1f}\n")
        fh.write(f"write_kib_per_dispatch: {w_k[0]:.1f}\n")
        fh.write(f"dispatches: {f_k[1]} {w_k[1]}\n")
        fh.write(f"copy_bytes: {COPY_PROBE_BYTES}\n")
        fh.write(f"copy_fetch_kib: {f_c[0]:.1f}\n")
        fh.write(f"copy_write_kib: {w_c[0]:.1f}\n")
    print(open(path).read())


def summarize_trace(run_dir: str):
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace run (CSV output)."""
    per = _trace_durations(run_dir)
    print(f"{'calls':>7} {'mean_us':>10} {'p10_us':>10} {'median_us':>10} {'p90_us':>10}  kernel")
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        n = len(v)
        print(f"{n:7d} {sum(v) / n / 1e3:10.2f} {v[n // 10] / 1e3:10.2f} {v[n // 2] / 1e3:10.2f} "
              f"{v[(9 * n) // 10] / 1e3:10.2f}  {name[:150]}")


def summarize_pmc(run_dirs, match: str = "gemm_"):
    """Mean per dispatch of every counter in rocprofv3 --pmc runs (CSV output),
    per kernel whose name contains `match`."""
    per = {}
    for d in run_dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if match not in r["Kernel_Name"]:
                        continue
                    k = per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], {})
                    key = (f, r["Dispatch_Id"])
                    k[key] = k.get(key, 0.0) + float(r["Counter_Value"])
    for name in sorted(per):
        print(name[:150])
        for c in sorted(per[name]):
            v = per[name][c]
            print(f"  {c:32s} {sum(v.values()) / len(v):14.6g}   ({len(v)} dispatches)")


def summarize_clock(run_dir: str, match: str = "gemm_", xcds: int = 8):
    """Shader clock during each layer kernel, from one rocprofv3 run that takes
    GRBM_GUI_ACTIVE with --pmc and the dispatch times with --kernel-trace: the
    counter (summed over the XCDs) divided by the XCD count is the kernel's
    busy cycles, and those over its traced duration are the clock."""
    cyc = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if match in r["Kernel_Name"] and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    key = (r["Kernel_Name"], r["Dispatch_Id"])
                    cyc[key] = cyc.get(key, 0.0) + float(r["Counter_Value"])
    dur = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if match in r["Kernel_Name"]:
                    dur[(r["Kernel_Name"], r["Dispatch_Id"])] = \
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = {}
    for key, c in cyc.items():
        if key in dur and dur[key] > 0:
            per.setdefault(key[0], []).append((c / xcds / dur[key], dur[key]))
    if not per:
        raise SystemExit(f"no dispatch under {run_dir} has both GRBM_GUI_ACTIVE and a trace span")
    out = {}
    for name in sorted(per):
        ghz = sorted(g for g, _ in per[name])
        us = sum(d for _, d in per[name]) / len(per[name]) / 1e3
        out[name] = (_median(ghz), ghz[0], ghz[-1], len(ghz), us)
        print(f"{name[:110]}\n  shader clock median {out[name][0]:.3f} GHz (min {ghz[0]:.3f}, "
              f"max {ghz[-1]:.3f}) over {len(ghz)} dispatches, mean duration {us:.2f} us")
    return out


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", default="bf16", choices=["bf16", "signed", "planes", "single", "w4"],
                    help="bf16: the layer from bf16 input; signed/planes: time the GEMM on "
                         "an activation pre-quantised by segquant_quantize_dualscale; single: the "
                         "single-scale W8A8 baseline from bf16 input; w4: W4A8 (4-bit weights)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch each step from Python")
    ap.add_argument("--no-all", action="store_true", help="skip the all_workloads summary")
    ap.add_argument("--no-producer", action="store_true",
                    help="skip the producer-fusion comparison (activation fused with quantisation)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured ceilings (matrix-core loop, streaming read)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="a few plain steps of --workload, then the copy probe (run under "
                         "rocprofv3 --pmc)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel duration statistics of a rocprofv3 kernel trace")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print the mean per dispatch of each counter of rocprofv3 --pmc runs, "
                         "per layer kernel")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the counter record of --workload from two --pmc-pass runs")
    ap.add_argument("--summarize-clock", metavar="DIR",
                    help="shader clock per layer kernel from a rocprofv3 run with --pmc "
                         "GRBM_GUI_ACTIVE and --kernel-trace")
    ap.add_argument("--ingest-trace", metavar="DIR",
                    help="write the kernel-trace record of --workload from a rocprofv3 "
                         "--kernel-trace run of the headline phase (--no-all --no-producer "
                         "--no-peaks --no-cpu-baseline)")
    ap.add_argument("--trace-command", default=None,
                    help="the traced command, for the record written by --ingest-trace")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.summarize_clock:
        summarize_clock(args.summarize_clock)
        return
    if args.ingest_trace:
        import segmented_dual_scale_amd as S
        import segmented_dual_scale_amd.workloads as W
        wl = W.WORKLOADS[args.workload]
        kernel = workload_kernel(S, wl, args.mode)
        cmd = args.trace_command or "(command not given)"
        ingest_trace(args.ingest_trace, args.workload, args.mode, kernel, cmd, args.steps)
        return
    if args.ingest_pmc:
        import segmented_dual_scale_amd as S
        import segmented_dual_scale_amd.workloads as W
        wl = W.WORKLOADS[args.workload]
        kernel = workload_kernel(S, wl, args.mode)
        cmd = f"python3 bench.py --workload {args.workload} --mode {args.mode} --pmc-pass"
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload, args.mode, kernel, cmd)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer is a single-GPU kernel library and this "
              "build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import segmented_dual_scale_amd as S
    from segmented_dual_scale_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    S.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)  # default priority

    if args.pmc_pass:
        layer = Layer(S, W, dev, args.workload, args.mode, rotate=False)
        with torch.cuda.stream(stream):
            for i in range(8):
                layer.step(i)
        torch.cuda.synchronize()
        layer.free()
        copy_probe(dev)
        print(f"pmc pass done: {layer.kernel} on {args.workload}, 8 dispatches; copy probe "
              f"{COPY_PROBE_BYTES} bytes", flush=True)
        return

    use_graph = not args.no_graph
    layer = Layer(S, W, dev, args.workload, args.mode)
    wl = layer.wl
    ms_per_step, steps = layer.time(stream, args.steps, args.warmup, use_graph)
    m = layer.metrics(ms_per_step)
    # the dominant kernel's own launch: the whole step, or the GEMM launch of
    # a two-launch step timed alone
    ms_kernel = ms_per_step if layer.launches == 1 else \
        layer.gemm_ms(stream, args.steps, args.warmup, use_graph)
    mk = layer.metrics(ms_kernel)
    roof = {"bound": mk["bound"], "achieved": mk["value"], "peak": mk["peak"], "unit": mk["unit"],
            "frac": mk["frac"], "traffic": None, "kernel": layer.kernel,
            "per_launch": {"alg_bytes": layer.alg_bytes(), "alg_int8_ops": alg_ops(wl),
                           "avg_us": ms_kernel * 1e3}}
    tt = read_trace(layer.kernel, wl.name, args.mode)
    if tt is not None:
        # the same kernel's dispatch durations under rocprofv3 (its own run)
        tt["frac_from_mean"] = layer.metrics(tt["mean_us"] * 1e-3)["frac"]
        tt["frac_from_median"] = layer.metrics(tt["median_us"] * 1e-3)["frac"]
        roof["trace"] = tt
    tr = read_traffic(layer.kernel, wl.name, args.mode)
    if tr is not None:
        roof["traffic"] = tr["bytes_per_launch"]
        roof["traffic_unit"] = "bytes per launch"
        roof["traffic_detail"] = tr
    R, launches = layer.R, layer.launches
    x_host, w_host = layer.x, layer.w
    layer.free()
    del layer
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": m["value"], "unit": m["unit"], "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded generators with the workload's shapes and polarity structure)",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N,
                   "k_segments": len(wl.kseg), "n_segments": len(wl.nseg),
                   "per_column_weight_scale": wl.per_column, "activation_input": args.mode,
                   "rotating_sets": R, "hip_graph": use_graph, "launches_per_step": launches,
                   "useful_2mnk_tops": alg_ops(wl) / 2 / (ms_per_step * 1e-3) / 1e12},
        "roofline": roof,
        "pages_latency": PAGES_LATENCY,
    }
    if not args.no_all:
        summary = {}
        for name in W.ORDER:
            lay = Layer(S, W, dev, name, args.mode)
            ms, n = lay.time(stream, 1, 10, use_graph, min_seconds=0.05)
            mm = lay.metrics(ms)
            summary[name] = {"value": mm["value"], "unit": mm["unit"], "bound": mm["bound"],
                             "frac": mm["frac"], "us_per_step": ms * 1e3, "steps": n,
                             "kernel": lay.kernel, "launches_per_step": lay.launches,
                             "M": lay.wl.M, "K": lay.wl.K, "N": lay.wl.N}
            if not args.no_cpu_baseline:  # the oracle on a bounded row sample, about 1 s
                cb = cpu_baseline(lay.wl, lay.x, lay.w, seconds=1.0)
                summary[name]["cpu_oracle"] = {
                    "value": cb["value"], "unit": cb["unit"], "cores": cb["cores"],
                    "rows": int(cb["sample"].split(" of ")[0]),
                    "gpu_over_cpu": mm["value"] / cb["value"]}
            if lay.launches == 2:
                gms = lay.gemm_ms(stream, 1, 10, use_graph, min_seconds=0.05)
                summary[name]["gemm_us_per_launch"] = gms * 1e3
                summary[name]["gemm_frac"] = lay.metrics(gms)["frac"]
                # the pages' single launch: the same call with the quantisation
                # fused into the GEMM (SEGQ_GEMM_FUSED_QUANT, no workspace)
                work, flags = lay.work, lay.flags
                lay.work, lay.flags = None, flags | S.SEGQ_GEMM_FUSED_QUANT
                msf, _ = lay.time(stream, 1, 10, use_graph, min_seconds=0.05)
                lay.work, lay.flags = work, flags
                summary[name]["single_launch_us_per_step"] = msf * 1e3
                summary[name]["single_launch_over_two"] = msf / ms
            lay.free()
            del lay
            torch.cuda.empty_cache()
            if args.mode == "bf16":
                # the single-scale baseline of the same layer: what DualScale costs
                lay = Layer(S, W, dev, name, "single")
                ms1, _ = lay.time(stream, 1, 10, use_graph, min_seconds=0.05)
                summary[name]["single_scale_us_per_step"] = ms1 * 1e3
                summary[name]["dualscale_over_single"] = ms / ms1
                lay.free()
                del lay
                torch.cuda.empty_cache()
                # W4A8: the same layer with 4-bit weights
                lay = Layer(S, W, dev, name, "w4")
                ms4, _ = lay.time(stream, 1, 10, use_graph, min_seconds=0.05)
                m4 = lay.metrics(ms4)
                summary[name]["w4a8"] = {"us_per_step": ms4 * 1e3, "value": m4["value"],
                                         "unit": m4["unit"], "frac": m4["frac"],
                                         "alg_bytes": lay.alg_bytes()}
                lay.free()
                del lay
                torch.cuda.empty_cache()
        line["all_workloads"] = summary
    if not args.no_producer:
        line["producer_fusion"] = producer_fusion(S, W, dev, stream)
    if not args.no_peaks:
        slab = (wl.K * wl.N // (2 if args.mode == "w4" else 1)) if roof["bound"] == "hbm" else 0  # the weight one call streams
        mp = measured_peaks(dev, stream, slab)
        line["measured_peaks"] = mp
        ref = mp["hbm_read_gbs"] if roof["bound"] == "hbm" else mp["int8_mfma_tops"]
        roof["frac_of_measured"] = roof["achieved"] / ref
        if slab:
            # a launch that only streams this call's weight, back to back
            roof["stream_floor_us"] = mp["hbm_stream_slab_us"]
            roof["over_stream_floor"] = roof["per_launch"]["avg_us"] / mp["hbm_stream_slab_us"]
        sus = mp.get("mfma_loop_sustained_tops")
        dat = mp.get("mfma_loop_data_tops")
        if roof["bound"] != "hbm" and sus:
            roof["frac_of_sustained_mfma"] = roof["achieved"] / sus
        if roof["bound"] != "hbm" and dat:
            roof["frac_of_data_mfma"] = roof["achieved"] / dat
        for v in line.get("all_workloads", {}).values():
            ref = mp["hbm_read_gbs"] if v["bound"] == "hbm" else mp["int8_mfma_tops"]
            v["frac_of_measured"] = v["value"] / ref
            if v["bound"] != "hbm" and sus:
                v["frac_of_sustained_mfma"] = v["value"] / sus
                if v.get("gemm_us_per_launch"):
                    v["gemm_frac_of_sustained_mfma"] = v["gemm_frac"] * PEAK_INT8_TOPS / sus
            if v["bound"] != "hbm" and dat:
                v["frac_of_data_mfma"] = v["value"] / dat
                if v.get("gemm_us_per_launch"):
                    v["gemm_frac_of_data_mfma"] = v["gemm_frac"] * PEAK_INT8_TOPS / dat
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, x_host, w_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
