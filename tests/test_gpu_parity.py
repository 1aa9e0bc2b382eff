"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: activation scales, int8 codes (both layouts), packed weights and
weight scales, and every per-segment int32 accumulator.  Within
|y - y_ref| <= 8e-3 |y_ref| + 1e-3 max|y_ref|: the bf16 output.
"""
import numpy as np
import pytest

import oracle
import segmented_dual_scale_amd as S
from segmented_dual_scale_amd import workloads as W
from gpu_common import (DEV, GpuLayer, OracleLayer, bf16_dev_to_f64, nan_filled_bf16,
                        rows_every_block, to_dev, to_dev_bf16, y_tolerance_ok)

pytestmark = pytest.mark.gpu


def _q_planes_from_dev(q, layout, M, K):
    q = q.cpu().numpy()
    if layout == S.SEGQ_Q_SIGNED:
        q = q[:, :K]
        return np.maximum(q, 0).astype(np.int8), np.minimum(q, 0).astype(np.int8)
    return q[0, :, :K].copy(), q[1, :, :K].copy()


# ----------------------------------------------------- activation side ----
ACT_CASES = [
    # M, K, kseg, kind
    (1, 64, [64], "gelu"),
    (37, 192, [64, 128], "blocks"),
    (300, 512, [64] * 8, "blocks"),
    (129, 1536, [1536], "silu"),
    (64, 1000, [512, 488], "gelu"),      # ragged K (last segment not 64-aligned)
    (5, 8200, [4096, 4104], "normal"),
    (70, 600, [64] * 9 + [24], "blocks"),   # ten segments, the last one 24 wide
    (2, 65600, [8192] * 8 + [64], "normal"),  # long rows, nine segments
    (17, 256, [256], "pos"),
    (17, 256, [256], "neg"),
]


@pytest.mark.parametrize("M,K,kseg,kind", ACT_CASES)
def test_calibrate_and_quantize_bitexact(M, K, kseg, kind):
    x, _ = W.make_custom(M, K, 16, seed=M + K, kind=kind, x_scale=2.0)
    ref_scales = np.stack(oracle.calibrate_amax(x, kseg))
    xd = to_dev_bf16(x)
    act = S.segquant_calibrate_amax(xd, kseg)
    assert np.array_equal(act.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))
    qp, qn = oracle.quantize_dualscale(x, kseg, ref_scales[2], ref_scales[3])
    for layout in (S.SEGQ_Q_SIGNED, S.SEGQ_Q_PLANES):
        q = S.segquant_quantize_dualscale(xd, act, kseg, layout)
        gp, gn = _q_planes_from_dev(q, layout, M, K)
        assert np.array_equal(gp, qp), f"q+ mismatch layout {layout}"
        assert np.array_equal(gn, qn), f"q- mismatch layout {layout}"


def test_calibrate_and_quantize_ragged_row_in_padded_buffer():
    """K = 1003 (not a multiple of 8) inside rows padded to 1008: the last
    partial 8-element piece is handled element by element, padding ignored."""
    import torch
    M, K = 9, 1003
    x, _ = W.make_custom(M, K, 16, seed=11, kind="gelu", x_scale=3.0)
    kseg = [512, 491]
    ref = np.stack(oracle.calibrate_amax(x, kseg))
    qp, qn = oracle.quantize_dualscale(x, kseg, ref[2], ref[3])
    pad = np.full((M, 1008), W.f32_to_bf16_bits(np.array([50.0], np.float32))[0], np.uint16)
    pad[:, :K] = x
    xd = to_dev_bf16(pad)[:, :K]
    act = S.segquant_calibrate_amax(xd, kseg)
    assert np.array_equal(act.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    for layout in (S.SEGQ_Q_SIGNED, S.SEGQ_Q_PLANES):
        q = S.segquant_quantize_dualscale(xd, act, kseg, layout)
        gp, gn = _q_planes_from_dev(q, layout, M, K)
        assert np.array_equal(gp, qp) and np.array_equal(gn, qn)


def test_quantize_saturates_static_scales_and_infinities():
    """Scales calibrated on one batch, applied to a batch with larger values
    and +-Inf: codes clamp at the ends of each half's range."""
    calib, _ = W.make_custom(16, 128, 16, seed=1, kind="normal")
    x = W.f32_to_bf16_bits(W.bf16_bits_to_f32(calib) * np.float32(3.0))
    x[0, :4] = W.f32_to_bf16_bits(np.array([np.inf, -np.inf, 1e30, -1e30], np.float32))
    sc = np.stack(oracle.calibrate_amax(calib, [128]))
    qp, qn = oracle.quantize_dualscale(x, [128], sc[2], sc[3])
    act = S.segquant_calibrate_amax(to_dev_bf16(calib), [128])
    q = S.segquant_quantize_dualscale(to_dev_bf16(x), act, [128], S.SEGQ_Q_PLANES)
    gp, gn = _q_planes_from_dev(q, S.SEGQ_Q_PLANES, 16, 128)
    assert np.array_equal(gp, qp) and np.array_equal(gn, qn)
    assert gp[0, :4].tolist() == [127, 0, 127, 0] and gn[0, :4].tolist() == [0, -128, 0, -128]


# -------------------------------------------------------- weight side ----
W_CASES = [
    # K, N, kseg, nseg, per_column
    (64, 16, [64], [16], False),
    (256, 768, [256], [256, 256, 256], False),
    (192, 48, [64, 128], None, True),
    (1536, 1536, [64] * 24, [1536], False),
    (640, 272, [128, 512], [16, 256], False),
]


@pytest.mark.parametrize("K,N,kseg,nseg,per_column", W_CASES)
def test_weight_quantize_pack_bitexact(K, N, kseg, nseg, per_column):
    g = np.random.default_rng(K + N)
    w = (g.standard_normal((K, N)) * np.exp(g.uniform(-3, 0, N))[None, :]).astype(np.float32)
    wq, ws = oracle.quantize_weight(w, kseg, nseg, per_column)
    wp, gws = S.segquant_quantize_weight(to_dev(w), kseg, nseg, per_column)
    assert np.array_equal(gws.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(S.segquant_unpack_weight(wp, K, N).cpu().numpy(), wq)


# ---------------------------------------------------------------- GEMM ----
GEMM_CASES = [
    # M, K, N, kseg, nseg, per_column, kind
    (1, 64, 16, [64], [16], False, "gelu"),
    (2, 1536, 576, [1536], [96] * 6, False, "silu"),
    (3, 256, 48, [64, 192], None, True, "blocks"),
    (8, 512, 112, [128, 384], None, True, "blocks"),   # largest M with both halves in one operand
    (5, 2048, 64, [64] * 32, [64], False, "blocks"),    # 32 segments, the full weight ring
    (9, 1024, 160, [1024], [160], False, "gelu"),       # smallest M with an operand per half
    # one K-segment, M <= 8, the streaming kernel's rings of 16, 32 and 32
    # slots (10, 25 and 32 k-tiles), odd numbers of n-tiles
    (8, 640, 48, [640], None, True, "gelu"),
    (3, 1600, 80, [1600], [80], False, "silu"),
    (1, 2048, 32, [2048], None, True, "normal"),
    (40, 320, 96, [320], None, True, "gelu"),           # one segment, odd number of k-tiles
    (70, 192, 400, [192], [400], False, "silu"),        # one segment, three k-tiles, ragged N
    (16, 640, 256, [64] * 10, [256], False, "blocks"),
    (17, 256, 272, [256], None, True, "gelu"),
    (77, 384, 768, [128, 256], [256] * 3, False, "gelu"),
    (200, 1536, 1536, [64] * 24, [1536], False, "blocks"),
    (333, 512, 320, [512], None, True, "gelu"),
    (257, 1024, 528, [256] * 4, [528], False, "gelu"),
    (130, 704, 64, [64, 128, 512], [32, 32], False, "normal"),
    (64, 256, 768, [256], [256, 256, 256], False, "pos"),
    (64, 256, 256, [128, 128], None, True, "neg"),
    # one segment on enough 64 x 384 tiles (26 x 5) to use them rather than
    # the 32 x 128 tiles of small grids: ragged rows, columns and k-tiles
    (1641, 320, 1904, [320], None, True, "gelu"),
]


def _ids(c):
    return f"M{c[0]}_K{c[1]}_N{c[2]}_S{len(c[3])}_{c[6]}"


@pytest.mark.parametrize("case", GEMM_CASES, ids=[_ids(c) for c in GEMM_CASES])
@pytest.mark.parametrize("mode", ["bf16", "signed", "planes"])
def test_gemm_parity(case, mode):
    import torch
    M, K, N, kseg, nseg, per_column, kind = case
    x, w = W.make_custom(M, K, N, seed=M * 7 + K + N, kind=kind, x_scale=2.0)
    ref = OracleLayer(x, w, kseg, nseg, per_column)
    gpu = GpuLayer(x, w, kseg, nseg, per_column)
    assert np.array_equal(gpu.act.cpu().numpy().view(np.uint32), ref.act.view(np.uint32))
    flag_sets = [S.SEGQ_GEMM_FORCE_TILE]
    if M <= 16:
        flag_sets.append(S.SEGQ_GEMM_FORCE_SMALLM)
    for flags in flag_sets:
        y, acc = gpu.run(mode, flags=flags, debug=True)
        assert np.array_equal(acc.cpu().numpy(), ref.acc), f"int32 accumulators, flags {flags}"
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
        assert ok, f"bf16 Y out of tolerance (flags {flags}): {nbad} elements, worst excess {worst}"
        # the production variant (no accumulator dump; it may combine the
        # segments in another fp32 order) is within the same tolerance
        y2, _ = gpu.run(mode, flags=flags, debug=False)
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y2), ref.y)
        assert ok, f"production Y out of tolerance (flags {flags}): {nbad} elements, worst {worst}"


# Shapes for which the library quantises first when given a workspace (six or
# more output column tiles): one segment (tiles of 384), every segment one
# k-step (tiles of 256), general segments with an end inside a stage.
QFIRST_CASES = [
    # M, K, N, kseg
    (300, 512, 2304, [512]),
    (133, 640, 1536, [64] * 10),
    (70, 1024, 1792, [320, 448, 256]),
]


@pytest.mark.parametrize("M,K,N,kseg", QFIRST_CASES)
def test_gemm_quantize_first_parity(M, K, N, kseg):
    """bf16 input with a workspace: one quantisation launch into the
    workspace, then the GEMM from the codes.  The workspace ends up holding
    the signed codes (so the two-launch path ran); accumulators bit-exact;
    Y within tolerance; the fused launch (no workspace) agrees likewise."""
    import torch
    x, w = W.make_custom(M, K, N, seed=M + N, kind="blocks", x_scale=2.0)
    ref = OracleLayer(x, w, kseg, None, True)
    gpu = GpuLayer(x, w, kseg, None, True)
    nb = S.segquant_gemm_workspace_bytes(M, N, K, kseg)
    assert nb == M * K
    for debug in (True, False):
        work = torch.full((nb + 64,), 0x55, dtype=torch.uint8, device=DEV)
        y, acc = gpu.run("bf16", debug=debug, workspace=work)
        codes = work[:nb].view(torch.int8).view(M, K).cpu().numpy()
        assert np.array_equal(np.maximum(codes, 0), ref.qp) and np.array_equal(np.minimum(codes, 0), ref.qn)
        assert np.all(work[nb:].cpu().numpy() == 0x55), "write past the asked-for workspace"
        if debug:
            assert np.array_equal(acc.cpu().numpy(), ref.acc)
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
        assert ok, f"quantise-first Y out of tolerance: {nbad} elements, worst excess {worst}"
    # too small a workspace, or the flag: the fused launch, which leaves it alone
    for work_bytes, flags in ((nb - 16, S.SEGQ_GEMM_AUTO), (nb, S.SEGQ_GEMM_FUSED_QUANT)):
        work = torch.full((work_bytes,), 0x55, dtype=torch.uint8, device=DEV)
        y, acc = gpu.run("bf16", debug=True, workspace=work, flags=flags)
        assert np.all(work.cpu().numpy() == 0x55)
        assert np.array_equal(acc.cpu().numpy(), ref.acc)
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
        assert ok, f"fused Y out of tolerance: {nbad} elements, worst excess {worst}"


# ------------------------------------------------- single-scale mode ----
SINGLE_CASES = [
    # M, K, N, kseg, kind
    (2, 1536, 576, [1536], "silu"),            # streaming small-M kernel, both halves in one operand
    (12, 640, 256, [64] * 10, "blocks"),       # streaming small-M kernel, ten segments
    (333, 512, 320, [512], "gelu"),            # tile kernel, one segment
    (77, 384, 768, [128, 256], "gelu"),        # bf16: tile kernel, segments ending on whole stages;
                                               # codes: the LDS-staged kernel (eight-wave tiles)
    (130, 704, 64, [64, 128, 512], "normal"),  # bf16: tile kernel, a segment ending inside a stage;
                                               # codes: the LDS-staged kernel
    (200, 1536, 1536, [64] * 24, "blocks"),    # tile kernel, one k-step per segment; quantise-first
    (300, 512, 2304, [512], "gelu"),           # tile kernel, one segment, quantise-first
    (1641, 320, 1904, [320], "gelu"),          # tile kernel, one segment on 64 x 384 tiles
]


@pytest.mark.parametrize("case", SINGLE_CASES, ids=[f"M{c[0]}_K{c[1]}_N{c[2]}_S{len(c[3])}" for c in SINGLE_CASES])
@pytest.mark.parametrize("mode", ["bf16", "signed"])
def test_single_scale_parity(case, mode):
    """Single-scale W8A8 (SEGQ_GEMM_SINGLE_SCALE with the single-scale
    table): table bit-exact; the one product per segment (dumped in plane 0)
    equals the oracle's A+ + A- bit-exact; plane 1 untouched; Y within
    tolerance, with and without the dump."""
    import torch
    M, K, N, kseg, kind = case
    x, w = W.make_custom(M, K, N, seed=M + K + N, kind=kind, x_scale=2.0)
    s, s2, inv, inv2 = oracle.calibrate_amax_single(x, kseg)
    wq, ws = oracle.quantize_weight(w, kseg, None, True)
    qp, qn = oracle.quantize_dualscale(x, kseg, inv, inv2)
    acc_ref = oracle.segment_acc(qp, qn, wq, kseg)
    y_ref = oracle.dequantize(acc_ref, s, s2, ws)
    xd = to_dev_bf16(x)
    act = S.segquant_calibrate_amax_single(xd, kseg)
    ref_tab = np.stack([s, s2, inv, inv2])
    assert np.array_equal(act.cpu().numpy().view(np.uint32), ref_tab.view(np.uint32))
    wp, gws = S.segquant_quantize_weight(to_dev(w), kseg, None, True)
    xq = S.segquant_quantize_dualscale(xd, act, kseg, S.SEGQ_Q_SIGNED) if mode == "signed" else None
    for debug in (True, False):
        acc = (torch.full((2, len(kseg), M, N), -7, dtype=torch.int32, device=DEV)
               if debug else None)
        if mode == "bf16":
            y = S.segquant_gemm_w8a8_seg(xd, wp, gws, act, kseg, acc_debug=acc,
                                         flags=S.SEGQ_GEMM_SINGLE_SCALE)
        else:
            y = S.segquant_gemm_w8a8_seg(None, wp, gws, act, kseg, N=N, xq=xq,
                                         q_layout=S.SEGQ_Q_SIGNED, acc_debug=acc,
                                         flags=S.SEGQ_GEMM_SINGLE_SCALE)
        torch.cuda.synchronize()
        if debug:
            a = acc.cpu().numpy()
            assert np.array_equal(a[0], acc_ref[0] + acc_ref[1]), "single-scale product differs"
            assert np.all(a[1] == -7), "plane 1 was written"
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), y_ref)
        assert ok, f"single-scale Y out of tolerance (debug={debug}): {nbad} elements, worst {worst}"


@pytest.mark.parametrize("M,K,N,kseg", [(77, 384, 768, [128, 256]), (5, 512, 160, [512]),
                                         (200, 1536, 1536, [64] * 24)])
@pytest.mark.parametrize("mode", ["bf16", "signed"])
def test_halves_choice_on_nonnegative_input(M, K, N, kseg, mode):
    """A DualScale table with no negative half (calibrated on input >= 0):
    segquant_gemm_halves picks the one-product GEMM, which then gives the
    DualScale result exactly: plane 0 equals the oracle's A+ and the oracle's
    A- is zero; plane 1 untouched; Y within tolerance of the DualScale Y.  On
    input with negative values the choice is both halves."""
    import torch
    x, w = W.make_custom(M, K, N, seed=M + 3 * K + N, kind="pos", x_scale=2.0)
    ref = OracleLayer(x, w, kseg, None, True)
    assert not ref.acc[1].any()
    gpu = GpuLayer(x, w, kseg, None, True)
    flags = S.segquant_gemm_halves(gpu.act)
    assert flags == S.SEGQ_GEMM_SINGLE_SCALE
    y, acc = gpu.run(mode, flags=flags, debug=True)
    a = acc.cpu().numpy()
    assert np.array_equal(a[0], ref.acc[0]), "one product differs from the + half's"
    assert np.all(a[1] == -7), "plane 1 was written"
    ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
    assert ok, f"Y out of tolerance: {nbad} elements, worst excess {worst}"
    xg, _ = W.make_custom(M, K, N, seed=M + 3 * K + N, kind="gelu", x_scale=2.0)
    assert S.segquant_gemm_halves(S.segquant_calibrate_amax(to_dev_bf16(xg), kseg)) == 0


@pytest.mark.parametrize("M", [2, 40])
@pytest.mark.parametrize("mode", ["bf16", "signed"])
@pytest.mark.parametrize("nk", [1, 4])
def test_gemm_at_the_int32_bound(M, mode, nk):
    """K = 132096 (the largest multiple of 64 within SEGQ_MAX_KSEG_WIDTH) in
    one K-segment, or four (on bf16 input the tile kernel's int32 running
    sums then span all of K; on codes the LDS-staged kernel folds each
    segment's own sums), with operands that put every accumulator at its largest
    magnitude: rows of -1 quantise to -128 throughout, rows of +1 to 127,
    columns of -0.02 / +0.02 to -127 / 127, so one segment's A- reaches
    132096 * 128 * 127 = 2147352576 (2^31 - 131072).  The chunked small-M
    kernel (M = 2) and the tile kernel (M = 40): accumulators bit-exact, Y
    within tolerance."""
    K, N = 132096, 32
    kseg = [K // nk] * nk
    x = np.ones((M, K), np.float32)
    x[0::2] = -1.0
    g = np.random.default_rng(7)
    if M > 4:
        x[4:8] = g.uniform(-1.0, 1.0, (4, K)).astype(np.float32)  # mixed rows within the range
    w = np.full((K, N), 0.02, np.float32)
    w[:, 0::2] = -0.02
    w[:, 8:12] = (g.standard_normal((K, 4)) * 0.02).astype(np.float32)
    xb = W.f32_to_bf16_bits(x)
    ref = OracleLayer(xb, w, kseg, None, True)
    assert int(np.abs(ref.acc.astype(np.int64)).max()) == (K // nk) * 128 * 127
    gpu = GpuLayer(xb, w, kseg, None, True)
    y, acc = gpu.run(mode, debug=True)
    assert np.array_equal(acc.cpu().numpy(), ref.acc)
    ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
    assert ok, f"Y out of tolerance: {nbad} elements, worst excess {worst}"


@pytest.mark.parametrize("M", [2, 40])
@pytest.mark.parametrize("mode", ["bf16", "signed", "planes", "single"])
def test_gemm_k_beyond_the_int32_bound_in_segments(M, mode):
    """K = 264192, twice SEGQ_MAX_KSEG_WIDTH's multiple of 64, as two
    K-segments of 132096, each driven to its own int32 limit (the operands of
    test_gemm_at_the_int32_bound): only each segment's sums must fit in int32
    ([P1] "SegLinear", input-segmented sum of per-segment products), so every
    per-segment accumulator is exact although their total is not an int32.
    Streaming small-M kernel (M = 2) and the large-M kernel that folds each
    segment's own sums (M = 40), every input mode and the single-scale
    product; accumulators bit-exact, Y within tolerance."""
    K1, N = 132096, 32
    kseg = [K1, K1]
    K = 2 * K1
    x = np.ones((M, K), np.float32)
    x[0::2] = -1.0
    g = np.random.default_rng(11)
    if M > 4:
        x[4:8] = g.uniform(-1.0, 1.0, (4, K)).astype(np.float32)
    w = np.full((K, N), 0.02, np.float32)
    w[:, 0::2] = -0.02
    w[:, 8:12] = (g.standard_normal((K, 4)) * 0.02).astype(np.float32)
    xb = W.f32_to_bf16_bits(x)
    gpu = GpuLayer(xb, w, kseg, None, True)
    if mode == "single":
        import torch
        s1, s2, inv, inv2 = oracle.calibrate_amax_single(xb, kseg)
        wq, ws = oracle.quantize_weight(w, kseg, None, True)
        qp, qn = oracle.quantize_dualscale(xb, kseg, inv, inv2)
        acc_ref = oracle.segment_acc(qp, qn, wq, kseg)
        y_ref = oracle.dequantize(acc_ref, s1, s2, ws)
        act = S.segquant_calibrate_amax_single(gpu.xd, kseg)
        xq = S.segquant_quantize_dualscale(gpu.xd, act, kseg, S.SEGQ_Q_SIGNED)
        for src in ("bf16", "signed"):
            acc = torch.full((2, len(kseg), M, N), -7, dtype=torch.int32, device=DEV)
            if src == "bf16":
                y = S.segquant_gemm_w8a8_seg(gpu.xd, gpu.wp, gpu.ws, act, kseg, acc_debug=acc,
                                             flags=S.SEGQ_GEMM_SINGLE_SCALE)
            else:
                y = S.segquant_gemm_w8a8_seg(None, gpu.wp, gpu.ws, act, kseg, xq=xq, N=N,
                                             acc_debug=acc, flags=S.SEGQ_GEMM_SINGLE_SCALE)
            a = acc.cpu().numpy()
            assert np.array_equal(a[0], acc_ref[0] + acc_ref[1]), f"single-scale products ({src})"
            assert np.all(a[1] == -7), f"plane 1 was written ({src})"
            ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), y_ref)
            assert ok, f"single-scale Y ({src}): {nbad} elements, worst excess {worst}"
        return
    ref = OracleLayer(xb, w, kseg, None, True)
    assert int(np.abs(ref.acc.astype(np.int64)).max()) == K1 * 128 * 127
    assert int(np.abs(ref.acc.astype(np.int64).sum(axis=1)).max()) > 2**31 - 1
    y, acc = gpu.run(mode, debug=True)
    assert np.array_equal(acc.cpu().numpy(), ref.acc)
    ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
    assert ok, f"Y out of tolerance: {nbad} elements, worst excess {worst}"
    y2, _ = gpu.run(mode, debug=False)
    assert np.array_equal(bf16_dev_to_f64(y2), bf16_dev_to_f64(y))


@pytest.mark.parametrize("M", [3, 40])
@pytest.mark.parametrize("mode", ["bf16", "signed", "planes"])
@pytest.mark.parametrize("case", ["x_zero", "w_zero", "one_segment_zero", "one_group_zero"])
def test_gemm_zero_ranges(M, mode, case):
    """Zero ranges (s = 0 and inv = 0, so that half or group is all zero
    codes): an all-zero activation or weight gives Y = 0 exactly; a zero
    K-segment of X, or a zero weight group, contributes nothing beside the
    others.  Scales and accumulators bit-exact, Y within tolerance (exact
    zeros where the whole output is zero)."""
    K, N, kseg, nseg = 512, 96, [128, 256, 128], [32, 32, 32]
    x, w = W.make_custom(M, K, N, seed=M + len(case), kind="gelu", x_scale=2.0)
    xf = W.bf16_bits_to_f32(x)
    if case == "x_zero":
        xf[:] = 0.0
    elif case == "one_segment_zero":
        xf[:, 128:384] = 0.0
    elif case == "w_zero":
        w[:] = 0.0
    else:
        w[128:384, 32:64] = 0.0  # K-segment 1 x N-segment 1: one weight group
    x = W.f32_to_bf16_bits(xf)
    ref = OracleLayer(x, w, kseg, nseg, False)
    gpu = GpuLayer(x, w, kseg, nseg, False)
    assert np.array_equal(gpu.act.cpu().numpy().view(np.uint32), ref.act.view(np.uint32))
    assert np.array_equal(gpu.ws.cpu().numpy().view(np.uint32), ref.ws.view(np.uint32))
    y, acc = gpu.run(mode, debug=True)
    assert np.array_equal(acc.cpu().numpy(), ref.acc)
    yg = bf16_dev_to_f64(y)
    if case in ("x_zero", "w_zero"):
        assert not ref.y.any() and not yg.any(), "the output is not exactly zero"
    ok, worst, nbad = y_tolerance_ok(yg, ref.y)
    assert ok, f"Y out of tolerance: {nbad} elements, worst excess {worst}"


def test_gemm_empty_batch_is_a_noop():
    import torch
    x, w = W.make_custom(4, 128, 32, seed=3)
    gpu = GpuLayer(x, w, [128], [32], False)
    empty = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    y = S.segquant_gemm_w8a8_seg(empty, gpu.wp, gpu.ws, gpu.act, [128])
    assert tuple(y.shape) == (0, 32)


def test_gemm_does_not_write_outside_its_rows():
    """Rows of a larger Y buffer outside [0, M) and columns beyond N keep
    their contents (guard bands)."""
    import torch
    M, K, N = 77, 256, 272
    x, w = W.make_custom(M, K, N, seed=5, kind="gelu")
    ref = OracleLayer(x, w, [256], None, True)
    gpu = GpuLayer(x, w, [256], None, True)
    for flags in (S.SEGQ_GEMM_FORCE_TILE,):
        big = torch.full((M + 3, N + 32), 7.0, dtype=torch.bfloat16, device=DEV)
        out = big[1:M + 1, :N]
        S.segquant_gemm_w8a8_seg(gpu.xd, gpu.wp, gpu.ws, gpu.act, [256], out=out, flags=flags)
        torch.cuda.synchronize()
        b = big.float().cpu().numpy()
        assert np.all(b[0] == 7.0) and np.all(b[M + 1:] == 7.0) and np.all(b[:, N:] == 7.0)
        ok, worst, nbad = y_tolerance_ok(b[1:M + 1, :N].astype(np.float64), ref.y)
        assert ok


@pytest.mark.parametrize("M,K,N,kseg", [(3, 512, 160, [512]),            # streaming small-M
                                         (5, 4096, 64, [2048, 2048]),     # chunked small-M
                                         (77, 384, 272, [128, 256]),      # tile, fused
                                         (150, 512, 2304, [512])])        # tile, quantise-first
@pytest.mark.parametrize("mode", ["bf16", "signed", "planes"])
def test_gemm_padded_operands_and_guard_bands(M, K, N, kseg, mode):
    """X (or its codes) inside a padded buffer (ld_x = K + 72, ld_q = K +
    48) and Y inside a larger one (rows above and below, 24 columns to the
    right): the result equals the oracle's (accumulators bit-exact) and no
    byte of Y's buffer outside the M x N window changes."""
    import torch
    x, w = W.make_custom(M, K, N, seed=M + K, kind="gelu", x_scale=2.0)
    ref = OracleLayer(x, w, kseg, None, True)
    gpu = GpuLayer(x, w, kseg, None, True)
    xpad = np.zeros((M, K + 72), np.uint16)
    xpad[:, :K] = x
    xd = to_dev_bf16(xpad)[:, :K]
    big = torch.full((M + 5, N + 24), 7.0, dtype=torch.bfloat16, device=DEV)
    out = big[2:M + 2, :N]
    acc = torch.full((2, len(kseg), M, N), -7, dtype=torch.int32, device=DEV)
    if mode == "bf16":
        S.segquant_gemm_w8a8_seg(xd, gpu.wp, gpu.ws, gpu.act, kseg, out=out, acc_debug=acc)
    else:
        lay = S.SEGQ_Q_SIGNED if mode == "signed" else S.SEGQ_Q_PLANES
        ldq = K + 48
        qbuf = torch.zeros((M, ldq) if mode == "signed" else (2, M, ldq), dtype=torch.int8,
                           device=DEV)
        S.segquant_quantize_dualscale(xd, gpu.act, kseg, lay, out=qbuf)
        S.segquant_gemm_w8a8_seg(None, gpu.wp, gpu.ws, gpu.act, kseg, N=N, xq=qbuf, q_layout=lay,
                                 out=out, acc_debug=acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), ref.acc)
    b = big.float().cpu().numpy()
    assert np.all(b[:2] == 7.0) and np.all(b[M + 2:] == 7.0) and np.all(b[:, N:] == 7.0)
    ok, worst, nbad = y_tolerance_ok(b[2:M + 2, :N].astype(np.float64), ref.y)
    assert ok, f"Y out of tolerance: {nbad} elements, worst excess {worst}"


# ------------------------------------------- full-size named workloads ----
@pytest.mark.parametrize("name", W.ORDER)
def test_full_size_workload(name):
    """At the workloads' full sizes and in the configuration the benchmark
    times: scales, packed weights bit-exact; int32 accumulators and Y on the
    first and last 8 rows and one random row of every 32-row block (so every
    row tile of the kernel, the ragged last one included); Y prefilled with
    NaN, so an element of the whole M x N output that no tile writes fails."""
    import torch
    wl, x, w = W.make_inputs(name)
    nseg = None if wl.per_column else list(wl.nseg)
    rows = rows_every_block(wl.M) if wl.M > 64 else np.arange(wl.M)
    ref = OracleLayer(x, w, wl.kseg, nseg, wl.per_column, rows=rows, with_acc=True)
    gpu = GpuLayer(x, w, wl.kseg, nseg, wl.per_column)
    assert np.array_equal(gpu.act.cpu().numpy().view(np.uint32), ref.act.view(np.uint32))
    assert np.array_equal(gpu.ws.cpu().numpy().view(np.uint32), ref.ws.view(np.uint32))
    assert np.array_equal(S.segquant_unpack_weight(gpu.wp, wl.K, wl.N).cpu().numpy(), ref.wq)
    ymax = float(np.abs(ref.y).max())
    ridx = torch.from_numpy(rows).to(DEV)
    # as the benchmark calls it (a workspace when the library asks for one),
    # and the fused launch
    for flags in (S.SEGQ_GEMM_AUTO, S.SEGQ_GEMM_FUSED_QUANT):
        y, _ = gpu.run("bf16", debug=False, flags=flags, out=nan_filled_bf16(wl.M, wl.N))
        assert not bool(torch.isnan(y).any()), f"{name} flags {flags}: output elements left unwritten"
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y)[rows], ref.y, ymax)
        assert ok, f"{name} flags {flags}: {nbad} sampled outputs out of tolerance, worst {worst}"
        yd, acc = gpu.run("bf16", debug=True, flags=flags, out=nan_filled_bf16(wl.M, wl.N))
        assert not bool(torch.isnan(yd).any()), \
            f"{name} flags {flags}: accumulator-dumping variant left output elements unwritten"
        acc_rows = acc.index_select(2, ridx).cpu().numpy()
        del acc
        assert np.array_equal(acc_rows, ref.acc), f"{name} flags {flags}: int32 accumulators differ"
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(yd)[rows], ref.y, ymax)
        assert ok, f"{name} flags {flags}: accumulator-dumping variant out of tolerance, worst {worst}"


# --------------------------------------- segments discovered from a graph ----
def test_discovered_segments_drive_the_layer():
    """The segment lists read off a module's graph (SegLinear discovery) go
    straight into the layer: an attention output projection (K-segments per
    head) and an AdaNorm projection (N-segments per modulation vector), each
    run through the kernels and compared with the oracle on the same lists."""
    import torch
    from segmented_dual_scale_amd import seglinear

    class AttnOut(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.proj = torch.nn.Linear(4 * 64, 256)

        def forward(self, o):
            b, h, t, d = o.shape
            return self.proj(o.transpose(1, 2).reshape(b, t, h * d))

    class AdaNorm(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.lin = torch.nn.Linear(256, 6 * 256)

        def forward(self, e):
            return self.lin(torch.nn.functional.silu(e)).chunk(6, dim=-1)

    torch.manual_seed(0)
    for mod, example, M in ((AttnOut(), torch.randn(1, 4, 3, 64), 150),
                            (AdaNorm(), torch.randn(2, 256), 2)):
        plan = next(iter(seglinear.discover(mod, example).values()))
        assert plan.kernel_ready()
        lin = mod.proj if isinstance(mod, AttnOut) else mod.lin
        K, N = lin.in_features, lin.out_features
        kseg = plan.kseg or [K]
        nseg = plan.nseg or [N]
        w = lin.weight.detach().t().contiguous().numpy().astype(np.float32)   # Y = X W, W [K][N]
        x, _ = W.make_custom(M, K, 16, seed=M, kind="gelu", x_scale=2.0)
        ref = OracleLayer(x, w, kseg, nseg, False)
        gpu = GpuLayer(x, w, kseg, nseg, False)
        y, acc = gpu.run("bf16", debug=True)
        assert np.array_equal(acc.cpu().numpy(), ref.acc)
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), ref.y)
        assert ok, f"{type(mod).__name__}: {nbad} outputs out of tolerance, worst {worst}"


# ------------------------------------- producer fused with quantisation ----
ACTQ_CASES = [
    # M, K, kseg, activation, z scale
    (37, 512, [512], "gelu", 3.0),
    (64, 1000, [512, 488], "silu", 2.0),      # ragged K: element-wise tail
    (300, 1536, [64] * 24, "gelu", 1.5),
    (5, 8200, [4096, 4104], "silu", 4.0),
]


@pytest.mark.parametrize("case", ACTQ_CASES, ids=[f"M{c[0]}_K{c[1]}_{c[3]}" for c in ACTQ_CASES])
@pytest.mark.parametrize("layout", [S.SEGQ_Q_SIGNED, S.SEGQ_Q_PLANES])
def test_activate_quantize_parity(case, layout):
    """SiLU/GELU fused with the quantisation.  The bf16 activation the
    kernel produces lies, element by element, between the bf16 roundings of
    the fp64 activation minus and plus a bound on fp32 evaluation error
    (2^-19 |act(z)|, a few fp32 ulps; bf16 spacing is 2^-8), and differs
    from the rounding of the fp64 value in under 0.1 % of elements; its codes equal the
    oracle's quantisation of those same bf16 values bit for bit; the
    calibration on them is bit-exact; codes alone equal codes with the copy."""
    import torch
    M, K, kseg, kind, scale = case
    z, _ = W.make_custom(M, K, 16, seed=K + M, kind="normal", x_scale=scale)
    act_kind = S.SEGQ_ACT_SILU if kind == "silu" else S.SEGQ_ACT_GELU
    zd = to_dev_bf16(z)
    _, xdev = S.segquant_activate_quantize(zd, act_kind, kseg=kseg, x_out=True, want_codes=False)
    torch.cuda.synchronize()
    xb = xdev.view(torch.int16).cpu().numpy().view(np.uint16)
    v = oracle.activation(z, kind)
    delta = 2.0 ** -19 * np.abs(v) + 2.0 ** -140
    lo = W.bf16_bits_to_f32(W.f32_to_bf16_bits((v - delta).astype(np.float32)))
    hi = W.bf16_bits_to_f32(W.f32_to_bf16_bits((v + delta).astype(np.float32)))
    xf = W.bf16_bits_to_f32(xb)
    assert np.all((xf >= lo) & (xf <= hi)), "activation outside its error bound"
    exact = W.bf16_bits_to_f32(W.f32_to_bf16_bits(v.astype(np.float32)))
    assert np.mean(xf != exact) < 1e-3
    # calibration on the produced values, then the fused codes
    act = S.segquant_calibrate_amax(xdev, kseg)
    sp, sn, ip, ineg = oracle.calibrate_amax(xb, kseg)
    assert np.array_equal(act.cpu().numpy().view(np.uint32),
                          np.stack([sp, sn, ip, ineg]).view(np.uint32))
    qp, qn = oracle.quantize_dualscale(xb, kseg, ip, ineg)
    q1, x2 = S.segquant_activate_quantize(zd, act_kind, act, kseg, layout, x_out=True)
    q2, _ = S.segquant_activate_quantize(zd, act_kind, act, kseg, layout)
    torch.cuda.synchronize()
    assert torch.equal(x2, xdev)
    for q in (q1, q2):
        gp, gn = _q_planes_from_dev(q, layout, M, K)
        assert np.array_equal(gp, qp) and np.array_equal(gn, qn), "fused codes differ"


@pytest.mark.parametrize("kind", ["silu", "gelu"])
def test_activation_every_bf16_input(kind):
    """Every finite bf16 value (65280 of them, as a 255 x 256 tensor) through
    the fused activation: each produced bf16 is finite and lies between the
    bf16 roundings of the fp64 activation minus and plus 2^-19 |act(z)| +
    2^-140, from the smallest subnormals to the largest magnitudes (where
    e^-z overflows and erfc underflows)."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    z = bits[np.isfinite(W.bf16_bits_to_f32(bits))].reshape(255, 256)
    act_kind = S.SEGQ_ACT_SILU if kind == "silu" else S.SEGQ_ACT_GELU
    _, xdev = S.segquant_activate_quantize(to_dev_bf16(z), act_kind, kseg=[256], x_out=True,
                                           want_codes=False)
    torch.cuda.synchronize()
    xf = W.bf16_bits_to_f32(xdev.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.all(np.isfinite(xf))
    v = oracle.activation(z, kind)
    delta = 2.0 ** -19 * np.abs(v) + 2.0 ** -140
    lo = W.bf16_bits_to_f32(W.f32_to_bf16_bits((v - delta).astype(np.float32)))
    hi = W.bf16_bits_to_f32(W.f32_to_bf16_bits((v + delta).astype(np.float32)))
    bad = ~((xf >= lo) & (xf <= hi))
    assert not bad.any(), f"{int(bad.sum())} inputs outside the bound, e.g. z={W.bf16_bits_to_f32(z[bad][:4])}"


# ------------------------------------------------------- 4-bit weights ----
W4_CASES = [
    # M, K, N, kseg, nseg, per_column, kind
    (2, 1536, 576, [1536], [96] * 6, False, "silu"),     # streaming small-M kernel reads 4-bit tiles
    (3, 256, 48, [64, 192], None, True, "blocks"),
    (8, 2048, 64, [64] * 32, [64], False, "blocks"),
    (16, 4096, 64, [4096], None, True, "gelu"),          # K past the streaming kernel: widened
    (77, 384, 768, [128, 256], [256] * 3, False, "gelu"),  # tile kernel: widened in the workspace
    (333, 512, 320, [512], None, True, "gelu"),
]


@pytest.mark.parametrize("case", W4_CASES, ids=[f"M{c[0]}_K{c[1]}_N{c[2]}_S{len(c[3])}" for c in W4_CASES])
@pytest.mark.parametrize("mode", ["bf16", "signed"])
def test_w4a8_parity(case, mode):
    """W4A8: 4-bit weight codes and scales bit-exact against the oracle's
    4-bit quantisation; per-segment accumulators bit-exact and Y within
    tolerance, on the streaming kernel (4-bit tiles read directly) and on
    the paths that widen them to int8 first."""
    import torch
    M, K, N, kseg, nseg, per_column, kind = case
    x, w = W.make_custom(M, K, N, seed=M + 7 * K, kind=kind, x_scale=2.0)
    sp, sn, ip, ineg = oracle.calibrate_amax(x, kseg)
    wq, ws = oracle.quantize_weight(w, kseg, nseg, per_column, bits=4)
    qp, qn = oracle.quantize_dualscale(x, kseg, ip, ineg)
    acc_ref = oracle.segment_acc(qp, qn, wq, kseg)
    y_ref = oracle.dequantize(acc_ref, sp, sn, ws)
    xd = to_dev_bf16(x)
    act = S.segquant_calibrate_amax(xd, kseg)
    wp, gws = S.segquant_quantize_weight(to_dev(w), kseg, nseg, per_column, bits=4)
    assert wp.numel() == K * N // 2
    assert np.array_equal(S.segquant_unpack_weight(wp, K, N, bits=4).cpu().numpy(), wq)
    assert np.array_equal(gws.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    xq = S.segquant_quantize_dualscale(xd, act, kseg, S.SEGQ_Q_SIGNED) if mode == "signed" else None
    for debug in (True, False):
        acc = (torch.full((2, len(kseg), M, N), -7, dtype=torch.int32, device=DEV)
               if debug else None)
        if mode == "bf16":
            y = S.segquant_gemm_w8a8_seg(xd, wp, gws, act, kseg, N=N, acc_debug=acc,
                                         flags=S.SEGQ_GEMM_W4)
        else:
            y = S.segquant_gemm_w8a8_seg(None, wp, gws, act, kseg, N=N, xq=xq,
                                         q_layout=S.SEGQ_Q_SIGNED, acc_debug=acc,
                                         flags=S.SEGQ_GEMM_W4)
        torch.cuda.synchronize()
        if debug:
            assert np.array_equal(acc.cpu().numpy(), acc_ref), "W4A8 accumulators differ"
        ok, worst, nbad = y_tolerance_ok(bf16_dev_to_f64(y), y_ref)
        assert ok, f"W4A8 Y out of tolerance (debug={debug}): {nbad} elements, worst {worst}"


# ------------------------------------------------------------ HIP graphs ----
@pytest.mark.parametrize("name", ["c2_adanorm_gemv", "c4_attn_out_inseg"])
def test_graph_replays_match_eager(name):
    """The layer captured in a HIP graph (the benchmark's timed form; for c4
    the two-launch quantise-first path with its workspace) and replayed
    several times, with eager work and synchronisations between replays:
    every replay's Y equals the eager call's bit for bit (same kernels, no
    memset nodes)."""
    import torch
    wl, x, w = W.make_inputs(name)
    nseg = None if wl.per_column else list(wl.nseg)
    gpu = GpuLayer(x, w, wl.kseg, nseg, wl.per_column)
    nb = S.segquant_gemm_workspace_bytes(wl.M, wl.N, wl.K, list(wl.kseg))
    work = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV) if nb else None
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=DEV)
    y_eager = S.segquant_gemm_w8a8_seg(gpu.xd, gpu.wp, gpu.ws, gpu.act, list(wl.kseg),
                                       workspace=work).clone()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        S.segquant_gemm_w8a8_seg(gpu.xd, gpu.wp, gpu.ws, gpu.act, list(wl.kseg), out=out,
                                 workspace=work)
    for rep in range(3):
        out.fill_(7.0)                            # eager work between replays
        junk = torch.randn(1 << 16, device=DEV).sum()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y_eager), f"{name}: replay {rep} differs from the eager call"
        del junk


def _replay_matches(run, out, y_eager, what):
    """Capture run() in a graph; replay three times with eager work and
    synchronisations between replays; every replay equals y_eager."""
    import torch
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run()
    for rep in range(3):
        out.fill_(7)                              # eager work between replays
        junk = torch.randn(1 << 16, device=DEV).sum()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y_eager), f"{what}: replay {rep} differs from the eager call"
        del junk


@pytest.mark.parametrize("name", ["c2_adanorm_gemv", "c3_dit_ffn_fc2"])
@pytest.mark.parametrize("variant", ["single", "w4"])
def test_graph_replays_of_variants(name, variant):
    """The single-scale layer and the W4A8 layer (on c3: the widening launch
    into the workspace, then the GEMM) captured and replayed: every replay
    equals the eager call bit for bit."""
    import torch
    wl, x, w = W.make_inputs(name)
    nseg = None if wl.per_column else list(wl.nseg)
    kseg = list(wl.kseg)
    xd = to_dev_bf16(x)
    if variant == "single":
        act = S.segquant_calibrate_amax_single(xd, kseg)
        wp, ws = S.segquant_quantize_weight(to_dev(w), kseg, nseg, wl.per_column)
        flags = S.SEGQ_GEMM_SINGLE_SCALE
    else:
        act = S.segquant_calibrate_amax(xd, kseg)
        wp, ws = S.segquant_quantize_weight(to_dev(w), kseg, nseg, wl.per_column, bits=4)
        flags = S.SEGQ_GEMM_W4
    nb = S.segquant_gemm_workspace_bytes(wl.M, wl.N, wl.K, kseg, flags=flags)
    work = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV) if nb else None
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=DEV)
    y_eager = S.segquant_gemm_w8a8_seg(xd, wp, ws, act, kseg, workspace=work, flags=flags).clone()
    torch.cuda.synchronize()
    _replay_matches(lambda: S.segquant_gemm_w8a8_seg(xd, wp, ws, act, kseg, out=out,
                                                     workspace=work, flags=flags),
                    out, y_eager, f"{name} {variant}")


@pytest.mark.parametrize("layout", ["signed", "planes"])
def test_graph_replays_of_activation_quantise(layout):
    """The fused GELU + dual-scale quantisation captured and replayed: the
    codes of every replay equal the eager call's."""
    import torch
    M, K, kseg = 600, 1536, [512, 1024]
    z, _ = W.make_custom(M, K, 16, seed=11, kind="normal", x_scale=2.0)
    zd = to_dev_bf16(z)
    lay = S.SEGQ_Q_SIGNED if layout == "signed" else S.SEGQ_Q_PLANES
    _, xdev = S.segquant_activate_quantize(zd, S.SEGQ_ACT_GELU, kseg=kseg, x_out=True,
                                           want_codes=False)
    act = S.segquant_calibrate_amax(xdev, kseg)
    q_eager, _ = S.segquant_activate_quantize(zd, S.SEGQ_ACT_GELU, act, kseg, lay)
    q_eager = q_eager.clone()
    out = torch.empty_like(q_eager)
    torch.cuda.synchronize()
    _replay_matches(lambda: S.segquant_activate_quantize(zd, S.SEGQ_ACT_GELU, act, kseg, lay,
                                                         out=out),
                    out, q_eager, f"activation quantise {layout}")

