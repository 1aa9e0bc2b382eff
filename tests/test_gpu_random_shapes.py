"""Seeded random layer shapes through the C ABI against the oracle.

The fixed cases elsewhere pin the paths one by one; these draws cover their
combinations.  Each case draws:
- M on either side of the kernels' tile edges and of the small-M limit;
- K in whole 64-wide k-tiles, with a random K-segment layout (boundaries on
  multiples of 64), sometimes every segment one k-step;
- N in multiples of 16, with random N-segments of any width, per-column
  weight scales, or one weight scale per K-segment;
- an input distribution and an activation input mode.

Bit-exact: the activation scales and every per-segment int32 accumulator (both
halves).  Within |y - y_ref| <= 8e-3 |y_ref| + 1e-3 max|y_ref|: the bf16 output,
with and without the accumulator dump.
"""
import numpy as np
import pytest

import segmented_dual_scale_amd as S
from segmented_dual_scale_amd import workloads as W
from gpu_common import GpuLayer, OracleLayer, bf16_dev_to_f64, y_tolerance_ok

pytestmark = pytest.mark.gpu

_MS = [1, 2, 3, 5, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 96, 127, 129, 200, 257, 311]
_KINDS = ["gelu", "silu", "normal", "pos", "neg", "blocks"]
_MODES = ["bf16", "signed", "planes"]


def _draw_cases(n: int = 48, seed: int = 20261203):
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(g.choice(_MS))
        kt = int(g.integers(1, 25))  # k-tiles of 64
        if kt > 1 and g.random() < 0.2:
            kseg = [64] * kt  # every segment one k-step
        else:
            ns = int(g.integers(1, min(kt, 6) + 1))
            cuts = sorted(g.choice(np.arange(1, kt), size=ns - 1, replace=False).tolist()) if ns > 1 else []
            edges = [0] + [64 * c for c in cuts] + [64 * kt]
            kseg = [b - a for a, b in zip(edges[:-1], edges[1:])]
        N = 16 * int(g.integers(1, 51))
        r = g.random()
        if r < 1 / 3:
            nseg, per_column = None, True
        elif r < 2 / 3:
            nseg, per_column = None, False
        else:
            nn = int(g.integers(1, min(N, 5) + 1))
            cuts = sorted(g.choice(np.arange(1, N), size=nn - 1, replace=False).tolist()) if nn > 1 else []
            edges = [0] + cuts + [N]
            nseg, per_column = [b - a for a, b in zip(edges[:-1], edges[1:])], False
        kind = str(g.choice(_KINDS))
        mode = str(g.choice(_MODES))
        cases.append((i, M, 64 * kt, N, kseg, nseg, per_column, kind, mode))
    return cases


CASES = _draw_cases()


def _id(c):
    i, M, K, N, kseg, nseg, per_column, kind, mode = c
    ns = "col" if per_column else (f"N{len(nseg)}" if nseg else "kseg")
    return f"{i:02d}_M{M}_K{K}_N{N}_S{len(kseg)}_{ns}_{kind}_{mode}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_parity(case):
    i, M, K, N, kseg, nseg, per_column, kind, mode = case
    x, w = W.make_custom(M, K, N, seed=1000 + i, kind=kind, x_scale=2.0)
    ref = OracleLayer(x, w, kseg, nseg, per_column)
    gpu = GpuLayer(x, w, kseg, nseg, per_column)
    assert np.array_equal(gpu.act.cpu().numpy().view(np.uint32), ref.act.view(np.uint32))
    flag_sets = [S.SEGQ_GEMM_AUTO]
    if M <= 16:  # both kernels take small M
        flag_sets.append(S.SEGQ_GEMM_FORCE_TILE)
    for flags in flag_sets:
        y, acc = gpu.run(mode, flags=flags, debug=True)
        assert np.array_equal(acc.cpu().numpy(), ref.acc), f"int32 accumulators, flags {flags}"
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
        assert ok, f"bf16 Y out of tolerance (flags {flags}): {nbad} elements, worst excess {worst}"
        y2, _ = gpu.run(mode, flags=flags, debug=False)
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y2), ref.y)
        assert ok, f"production Y out of tolerance (flags {flags}): {nbad} elements, worst {worst}"


def _draw_large(n: int = 12, seed: int = 20261204):
    """Larger M (several 128-row tiles and a ragged last one) and N (several
    column tiles and a ragged last one), several K-segments: the large-M
    kernels' tile edges, on every input mode and single-scale codes."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(g.integers(257, 700))
        kt = int(g.integers(2, 25))
        ns = int(g.integers(2, min(kt, 6) + 1))
        cuts = sorted(g.choice(np.arange(1, kt), size=ns - 1, replace=False).tolist())
        edges = [0] + [64 * c for c in cuts] + [64 * kt]
        kseg = [b - a for a, b in zip(edges[:-1], edges[1:])]
        N = 16 * int(g.integers(9, 49))
        per_column = bool(g.random() < 0.5)
        kind = str(g.choice(_KINDS))
        mode = ["bf16", "signed", "planes", "single"][i % 4]
        cases.append((i, M, 64 * kt, N, kseg, per_column, kind, mode))
    return cases


LARGE = _draw_large()


@pytest.mark.parametrize("case", LARGE, ids=[f"{c[0]:02d}_M{c[1]}_K{c[2]}_N{c[3]}_S{len(c[4])}_{c[7]}"
                                             for c in LARGE])
def test_random_large_shape_parity(case):
    """As above at larger M and N; "single" is the single-scale product on
    signed codes (one accumulator plane, equal to the oracle's A+ + A-)."""
    import torch
    import oracle
    i, M, K, N, kseg, per_column, kind, mode = case
    x, w = W.make_custom(M, K, N, seed=5000 + i, kind=kind, x_scale=2.0)
    if mode != "single":
        ref = OracleLayer(x, w, kseg, None, per_column)
        gpu = GpuLayer(x, w, kseg, None, per_column)
        for debug in (True, False):
            y, acc = gpu.run(mode, debug=debug)
            if debug:
                assert np.array_equal(acc.cpu().numpy(), ref.acc), "int32 accumulators"
            ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
            assert ok, f"Y out of tolerance (debug={debug}): {nbad} elements, worst excess {worst}"
        return
    s, s2, inv, inv2 = oracle.calibrate_amax_single(x, kseg)
    wq, ws = oracle.quantize_weight(w, kseg, None, per_column)
    qp, qn = oracle.quantize_dualscale(x, kseg, inv, inv2)
    acc_ref = oracle.segment_acc(qp, qn, wq, kseg)
    y_ref = oracle.dequantize(acc_ref, s, s2, ws)
    dev = "cuda:0"
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    act = S.segquant_calibrate_amax_single(xd, kseg)
    assert np.array_equal(act.cpu().numpy().view(np.uint32), np.stack([s, s2, inv, inv2]).view(np.uint32))
    wp, gws = S.segquant_quantize_weight(torch.from_numpy(w).to(dev), kseg, None, per_column)
    xq = S.segquant_quantize_dualscale(xd, act, kseg, S.SEGQ_Q_SIGNED)
    for debug in (True, False):
        acc = torch.full((2, len(kseg), M, N), -7, dtype=torch.int32, device=dev) if debug else None
        y = S.segquant_gemm_w8a8_seg(None, wp, gws, act, kseg, N=N, xq=xq, q_layout=S.SEGQ_Q_SIGNED,
                                     acc_debug=acc, flags=S.SEGQ_GEMM_SINGLE_SCALE)
        torch.cuda.synchronize()
        if debug:
            a = acc.cpu().numpy()
            assert np.array_equal(a[0], acc_ref[0] + acc_ref[1]), "single-scale product"
            assert np.all(a[1] == -7), "plane 1 was written"
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), y_ref)
        assert ok, f"single-scale Y out of tolerance (debug={debug}): {nbad} elements, worst {worst}"
