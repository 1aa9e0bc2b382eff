"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np

import oracle
import segmented_dual_scale_amd as S
from segmented_dual_scale_amd import workloads as W

DEV = "cuda:0"


def to_dev_bf16(xbits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(xbits).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def y_tolerance_ok(y: np.ndarray, yref: np.ndarray, ymax: float | None = None):
    """|y - y_ref| <= 8e-3 |y_ref| + 1e-3 max|y_ref| (max over the whole output)."""
    if ymax is None:
        ymax = float(np.abs(yref).max()) if yref.size else 0.0
    err = np.abs(y.astype(np.float64) - yref)
    bound = 8e-3 * np.abs(yref) + 1e-3 * ymax
    bad = err > bound
    return (not bad.any()), (float((err - bound).max()) if err.size else 0.0), int(bad.sum())


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64)


class OracleLayer:
    """Oracle side: calibration, weight quantisation, codes, per-segment
    accumulators and fp64 Y for (a subset of) the rows."""

    def __init__(self, x, w, kseg, nseg, per_column, rows=None, with_acc=True):
        self.kseg = list(kseg)
        self.sp, self.sn, self.ip, self.ineg = oracle.calibrate_amax(x, self.kseg)
        self.wq, self.ws = oracle.quantize_weight(w, self.kseg, nseg, per_column)
        xs = x if rows is None else np.ascontiguousarray(x[rows])
        if with_acc:
            self.qp, self.qn = oracle.quantize_dualscale(xs, self.kseg, self.ip, self.ineg)
            self.acc = oracle.segment_acc(self.qp, self.qn, self.wq, self.kseg)
            self.y = oracle.dequantize(self.acc, self.sp, self.sn, self.ws)
        else:
            self.y = oracle.dualscale_linear(xs, self.wq, self.ws, self.kseg, self.sp, self.sn,
                                             self.ip, self.ineg)

    @property
    def act(self):
        return np.stack([self.sp, self.sn, self.ip, self.ineg])


class GpuLayer:
    """HIP side through the C ABI."""

    def __init__(self, x, w, kseg, nseg, per_column):
        import torch
        self.kseg = list(kseg)
        self.xd = to_dev_bf16(x)
        wd = to_dev(w)
        self.M, self.K = x.shape
        self.N = w.shape[1]
        self.act = S.segquant_calibrate_amax(self.xd, self.kseg)
        self.wp, self.ws = S.segquant_quantize_weight(wd, self.kseg, nseg, per_column)
        del wd
        torch.cuda.synchronize()

    def run(self, mode="bf16", flags=S.SEGQ_GEMM_AUTO, debug=False, workspace="auto", out=None):
        import torch
        acc = None
        if debug:
            acc = torch.full((2, len(self.kseg), self.M, self.N), -7, dtype=torch.int32, device=DEV)
        if mode == "bf16":
            y = S.segquant_gemm_w8a8_seg(self.xd, self.wp, self.ws, self.act, self.kseg,
                                         acc_debug=acc, workspace=workspace, flags=flags, out=out)
        else:
            layout = S.SEGQ_Q_SIGNED if mode == "signed" else S.SEGQ_Q_PLANES
            xq = S.segquant_quantize_dualscale(self.xd, self.act, self.kseg, layout)
            y = S.segquant_gemm_w8a8_seg(None, self.wp, self.ws, self.act, self.kseg, xq=xq,
                                         q_layout=layout, N=self.N, acc_debug=acc, flags=flags,
                                         out=out)
        torch.cuda.synchronize()
        return y, acc


def rows_every_block(M: int, block: int = 32, seed: int = 0) -> np.ndarray:
    """The first and last 8 rows and one random row of every `block`-row
    block, sorted and unique.  Every row tile of the large-M kernels is a
    whole number of 32-row blocks, so each tile has a sampled row."""
    g = np.random.default_rng(seed)
    rows = set(range(min(8, M))) | set(range(max(0, M - 8), M))
    for b0 in range(0, M, block):
        rows.add(int(g.integers(b0, min(M, b0 + block))))
    return np.array(sorted(rows), dtype=np.int64)


def nan_filled_bf16(M: int, N: int):
    """A bf16 [M][N] device tensor holding a NaN in every element: an output
    element that a call leaves unwritten keeps it."""
    import torch
    return torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
