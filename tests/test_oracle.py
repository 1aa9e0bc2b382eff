"""Pins for the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula and compares: each checks the
oracle against a hand-derived example (arithmetic written out beside the
literal), an invariant of the definition, a special case that reduces to a
library routine (numpy integer/fp64 matmul), or brute force on tiny inputs.

Pages cited:
  [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
       for Diffusion Models" (papernotes.org, CVPR 2026 notes)
  [P2] "SegQuant" (hliangzhao.me/works/segquant.html)
"""
import math
import os

import numpy as np
import pytest

import oracle
from segmented_dual_scale_amd import workloads as W

bits = W.f32_to_bf16_bits
fl = W.bf16_bits_to_f32


def row(vals):
    return bits(np.array([vals], np.float32))


# ---------------------------------------------------------------- split ----
def test_polarity_split_exact():
    """[P1 DualScale, split equation]: X+ + X- = X exactly, X+ X- = 0."""
    g = np.random.default_rng(1)
    raw = g.integers(0, 1 << 16, 20000, dtype=np.uint16)
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x7F80, 0xFF80, 0x3F80, 0xBF80],
                       np.uint16)
    x = np.concatenate([raw, special])
    x = x[~np.isnan(fl(x))]
    xp, xn = oracle.polarity_split(x)
    xf = fl(x)
    fin = np.isfinite(xf)
    assert np.array_equal(xp[fin] + xn[fin], xf[fin])
    assert np.all(xp >= 0) and np.all(xn <= 0)
    assert np.all((xp == 0) | (xn == 0))
    # infinities land in the half of their sign
    assert np.array_equal(xp[~fin] + xn[~fin], xf[~fin])


# --------------------------------------------------- calibration + codes ----
def test_worked_example_e1():
    """Hand-derived from [P2 section 3] s+ = max/127, s- = |min|/128 and
    Q_dual, with q_max = 127, q_min = 128.

    x = [-0.28125, -0.0625, 0, 0.125, 3.5]
      s- = 0.28125/128 = 0.002197265625 (exact), inv- = 128/0.28125 = 455.11...
      s+ = 3.5/127, inv+ = 127/3.5 = 36.2857...
      -0.28125 * 455.11 = -128.000  -> -128     (the min maps to the end)
      -0.0625  * 455.11 =  -28.44   -> -28
       0.125   * 36.286 =    4.536  ->   5
       3.5     * 36.286 =  127.000  ->  127     (the max maps to the end)
    """
    x = row([-0.28125, -0.0625, 0.0, 0.125, 3.5])
    sp, sn, ip, ineg = oracle.calibrate_amax(x, [5])
    assert sn[0] == np.float32(0.002197265625)
    assert abs(float(sp[0]) - 3.5 / 127) < 1e-9
    assert abs(float(ip[0]) - 127 / 3.5) < 1e-5 and abs(float(ineg[0]) - 128 / 0.28125) < 1e-4
    qp, qn = oracle.quantize_dualscale(x, [5], ip, ineg)
    assert qp.tolist() == [[0, 0, 0, 5, 127]]
    assert qn.tolist() == [[-128, -28, 0, 0, 0]]


def test_worked_example_e2_ties_to_even():
    """Ties: max 63.5 gives s+ = 0.5 (inv+ = 2 exactly); min -64 gives
    s- = 0.5 (inv- = 2).  Products x*2 that are .5 ties:
      1.25 -> 2.5 -> 2,   0.75 -> 1.5 -> 2,   0.25 -> 0.5 -> 0,  1.75 -> 3.5 -> 4
     -1.25 -> -2,  -0.75 -> -2,  -0.25 -> 0,  -1.75 -> -4
    (half-away-from-zero would give 3, 2, 1, 4, -3, -2, -1, -4)."""
    x = row([63.5, -64.0, 1.25, 0.75, 0.25, 1.75, -1.25, -0.75, -0.25, -1.75])
    sp, sn, ip, ineg = oracle.calibrate_amax(x, [10])
    assert (sp[0], sn[0], ip[0], ineg[0]) == (0.5, 0.5, 2.0, 2.0)
    qp, qn = oracle.quantize_dualscale(x, [10], ip, ineg)
    assert qp.tolist() == [[127, 0, 2, 2, 0, 4, 0, 0, 0, 0]]
    assert qn.tolist() == [[0, -128, 0, 0, 0, 0, -2, -2, 0, -4]]


def test_saturation_and_infinities():
    """Static scales from one batch applied to larger values saturate at the
    code range ends ([0,127] and [-128,0]); +-Inf saturate too."""
    sp, sn, ip, ineg = oracle.calibrate_amax(row([1.0, -1.0]), [2])
    assert (ip[0], ineg[0]) == (127.0, 128.0)
    x = row([2.0, -2.0, np.inf, -np.inf, 1e30, -1e30, 0.5, -0.5])
    qp, qn = oracle.quantize_dualscale(x, [8], ip, ineg)
    # 0.5*127 = 63.5 -> 64 (tie to even);  -0.5*128 = -64
    assert qp.tolist() == [[127, 0, 127, 0, 127, 0, 64, 0]]
    assert qn.tolist() == [[0, -128, 0, -128, 0, -128, 0, -64]]


@pytest.mark.parametrize("kind,zero_half", [("pos", "neg"), ("neg", "pos")])
def test_zero_range_gives_zero_half(kind, zero_half):
    """A one-signed X has a zero range on the other side: s = inv = 0 and
    that half is identically zero (no 0*inf)."""
    x, _ = W.make_custom(7, 64, 16, seed=3, kind=kind)
    sp, sn, ip, ineg = oracle.calibrate_amax(x, [64])
    qp, qn = oracle.quantize_dualscale(x, [64], ip, ineg)
    if zero_half == "neg":
        assert sn[0] == 0 and ineg[0] == 0 and not qn.any() and qp.max() == 127
    else:
        assert sp[0] == 0 and ip[0] == 0 and not qp.any() and qn.min() == -128


def test_range_too_small_for_an_fp32_inverse_counts_as_zero():
    """127/a overflows fp32 for a below about 3.7e-37: such a range is
    treated like a zero range (s = inv = 0, codes 0), for activations and
    weights alike."""
    x = bits(np.array([[1e-38, -2.0, 0.0]], np.float32))
    sp, sn, ip, ineg = oracle.calibrate_amax(x, [3])
    assert (sp[0], ip[0]) == (0.0, 0.0) and sn[0] == np.float32(2.0 / 128)
    qp, qn = oracle.quantize_dualscale(x, [3], ip, ineg)
    assert qp.tolist() == [[0, 0, 0]] and qn.tolist() == [[0, -128, 0]]
    w = np.array([[1e-38, -1e-38], [0.0, 2.0]], np.float32)
    wq, ws = oracle.quantize_weight(np.repeat(w, 32, axis=0), [64], None, per_column=True)
    assert ws[0, 0] == 0 and not wq[:, 0].any()
    assert ws[0, 1] == np.float32(2.0 / 127) and wq[:, 1].min() == 0 and wq[:, 1].max() == 127


def test_signed_zero_and_subnormals():
    x = bits(np.array([[0.0, -0.0, 1e-40, -1e-40, 3.0, -3.0]], np.float32))
    sp, sn, ip, ineg = oracle.calibrate_amax(x, [6])
    qp, qn = oracle.quantize_dualscale(x, [6], ip, ineg)
    assert qp.tolist() == [[0, 0, 0, 0, 127, 0]]
    assert qn.tolist() == [[0, 0, 0, 0, 0, -128]]


def test_per_segment_scales_and_error_bound():
    """Input-segmented: each K-segment gets its own (s+, s-) from its own
    range (its max -> 127, its min -> -128), and for every unclamped element
    |x - s q| <= s/2 + 2^-21 |x| (the slack covers s*inv != 1 in fp32)."""
    x, _ = W.make_custom(33, 256, 16, seed=5, kind="blocks")
    kseg = [64, 128, 64]
    sp, sn, ip, ineg = oracle.calibrate_amax(x, kseg)
    qp, qn = oracle.quantize_dualscale(x, kseg, ip, ineg)
    xf = fl(x).astype(np.float64)
    off = 0
    for i, w in enumerate(kseg):
        sl = slice(off, off + w)
        seg = xf[:, sl]
        assert sp[i] == np.float32(seg.max() / 127) and sn[i] == np.float32(-seg.min() / 128)
        assert qp[:, sl][seg == seg.max()].tolist() == [127] * int((seg == seg.max()).sum())
        assert np.all(qn[:, sl][seg == seg.min()] == -128)
        pos = seg >= 0
        err_p = np.abs(seg[pos] - float(sp[i]) * qp[:, sl][pos])
        err_n = np.abs(seg[~pos] - float(sn[i]) * qn[:, sl][~pos])
        assert np.all(err_p <= float(sp[i]) / 2 + 2.0 ** -21 * np.abs(seg[pos]))
        assert np.all(err_n <= float(sn[i]) / 2 + 2.0 ** -21 * np.abs(seg[~pos]))
        off += w
    assert set(np.unique(qp)) <= set(range(0, 128))
    assert set(np.unique(qn)) <= set(range(-128, 1))
    assert not np.any((qp != 0) & (qn != 0))


@pytest.mark.parametrize("j", [-3, 5])
def test_power_of_two_scaling_invariance(j):
    """Scaling X by 2^j scales s by 2^j and inv by 2^-j exactly, so the
    codes do not change (no subnormals or overflow at these sizes)."""
    x, _ = W.make_custom(16, 128, 16, seed=9, kind="silu")
    x2 = bits(fl(x) * np.float32(2.0 ** j))
    a = oracle.calibrate_amax(x, [64, 64])
    b = oracle.calibrate_amax(x2, [64, 64])
    assert np.array_equal(b[0], a[0] * np.float32(2.0 ** j))
    assert np.array_equal(b[2], a[2] * np.float32(2.0 ** -j))
    qa = oracle.quantize_dualscale(x, [64, 64], a[2], a[3])
    qb = oracle.quantize_dualscale(x2, [64, 64], b[2], b[3])
    assert np.array_equal(qa[0], qb[0]) and np.array_equal(qa[1], qb[1])


# ------------------------------------------------------------- weights ----
def test_weight_groups_output_segmented():
    """[P1 SegLinear, output-segmented pattern]: each column segment is
    quantised on its own, so each segment's largest |w| maps to +-127 and
    its scale is its own amax/127, whatever the other segments hold."""
    g = np.random.default_rng(2)
    K, nseg = 128, [32, 64, 32]
    w = g.standard_normal((K, 128)).astype(np.float32)
    w[:, 32:96] *= 50.0
    wq, ws = oracle.quantize_weight(w, [K], nseg, per_column=False)
    off = 0
    for wd in nseg:
        blk, q = w[:, off:off + wd], wq[:, off:off + wd]
        a = np.abs(blk).max()
        assert np.all(ws[0, off:off + wd] == np.float32(a / 127.0))
        assert np.all(np.abs(q[np.abs(blk) == a]) == 127)
        s = float(ws[0, off])
        assert np.all(np.abs(blk - s * q) <= s / 2 + 2.0 ** -21 * np.abs(blk))
        off += wd
    assert wq.min() >= -127 and wq.max() <= 127


def test_weight_groups_input_segmented_and_per_column():
    """[P1 SegLinear, input-segmented pattern]: row segments get their own
    scale; with per_column each (row segment, column) has its own scale."""
    g = np.random.default_rng(4)
    K, N, kseg = 192, 48, [64, 128]
    w = g.standard_normal((K, N)).astype(np.float32)
    w[64:] *= 0.01
    wq, ws = oracle.quantize_weight(w, kseg, None, per_column=False)
    assert np.all(ws[0] == np.float32(np.abs(w[:64]).max() / 127))
    assert np.all(ws[1] == np.float32(np.abs(w[64:]).max() / 127))
    wq2, ws2 = oracle.quantize_weight(w, kseg, None, per_column=True)
    for i, (a, b) in enumerate([(0, 64), (64, 192)]):
        colmax = np.abs(w[a:b]).max(axis=0)
        assert np.array_equal(ws2[i], (colmax / 127.0).astype(np.float32))
        assert np.all(np.abs(wq2[a:b]).max(axis=0) == 127)


def test_weight_zero_group():
    w = np.zeros((64, 32), np.float32)
    w[:, 16:] = 1.0
    wq, ws = oracle.quantize_weight(w, [64], [16, 16], per_column=False)
    assert not wq[:, :16].any() and np.all(ws[0, :16] == 0)
    assert np.all(wq[:, 16:] == 127)


# ------------------------------------------------------------- products ----
def _brute_acc(qp, qn, wq, kseg):
    """Pure-Python triple loop on tiny inputs."""
    M, K = qp.shape
    N = wq.shape[1]
    out = np.zeros((2, len(kseg), M, N), np.int64)
    off = 0
    for i, wd in enumerate(kseg):
        for h, q in enumerate((qp, qn)):
            for m in range(M):
                for n in range(N):
                    s = 0
                    for k in range(off, off + wd):
                        s += int(q[m, k]) * int(wq[k, n])
                    out[h, i, m, n] = s
        off += wd
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_segment_acc_brute_force(seed):
    g = np.random.default_rng(seed)
    M, K, N = int(g.integers(1, 9)), 64 * int(g.integers(1, 4)), int(g.integers(1, 12))
    kseg = W.random_segments(K, g, align=16)
    qp = g.integers(0, 128, (M, K)).astype(np.int8)
    qn = g.integers(-128, 1, (M, K)).astype(np.int8)
    wq = g.integers(-127, 128, (K, N)).astype(np.int8)
    acc = oracle.segment_acc(qp, qn, wq, kseg)
    assert np.array_equal(acc, _brute_acc(qp, qn, wq, kseg))


def test_segment_acc_library_matmul_and_extremes():
    """Per-segment sums equal numpy int64 matmuls of the segment slices;
    one segment equals the unsegmented product; segment sums add up to it.
    Extreme codes (-128 x -127 over a 4096-wide segment) stay exact."""
    g = np.random.default_rng(7)
    M, K, N = 5, 4096 + 128, 24
    qp = g.integers(0, 128, (M, K)).astype(np.int8)
    qn = g.integers(-128, 1, (M, K)).astype(np.int8)
    qn[0, :] = -128
    wq = g.integers(-127, 128, (K, N)).astype(np.int8)
    wq[:, 0] = -127
    kseg = [4096, 64, 64]
    acc = oracle.segment_acc(qp, qn, wq, kseg)
    one = oracle.segment_acc(qp, qn, wq, [K])
    full_p = qp.astype(np.int64) @ wq.astype(np.int64)
    full_n = qn.astype(np.int64) @ wq.astype(np.int64)
    assert np.array_equal(one[0, 0], full_p) and np.array_equal(one[1, 0], full_n)
    assert np.array_equal(acc.astype(np.int64).sum(axis=1)[0], full_p)
    assert np.array_equal(acc.astype(np.int64).sum(axis=1)[1], full_n)
    assert acc[1, 0, 0, 0] == 4096 * 128 * 127
    off = 0
    for i, wd in enumerate(kseg):
        sl = slice(off, off + wd)
        assert np.array_equal(acc[0, i], qp[:, sl].astype(np.int64) @ wq[sl].astype(np.int64))
        off += wd


# ------------------------------------------------------- dequantisation ----
def _dequant_then_matmul(qp, qn, wq, ws, sp, sn, kseg):
    """The reconstruction written the other way round: dequantise each
    operand, then one fp64 library matmul (sum over k of x~ w~)."""
    M, K = qp.shape
    xs = np.zeros((M, K))
    wt = np.zeros(wq.shape)
    off = 0
    for i, wd in enumerate(kseg):
        sl = slice(off, off + wd)
        xs[:, sl] = float(sp[i]) * qp[:, sl] + float(sn[i]) * qn[:, sl]
        wt[sl] = wq[sl] * ws[i][None, :].astype(np.float64)
        off += wd
    return xs @ wt


@pytest.mark.parametrize("kseg,per_column", [([192], False), ([64, 64, 64], False),
                                             ([128, 64], True)])
def test_dequantize_matches_dequantised_operands(kseg, per_column):
    """[P1 DualScale reconstruction; P2 section 3]: y = s_w (s+ A+ + s- A-)
    summed over segments equals the product of the dequantised operands."""
    x, w = W.make_custom(19, 192, 40, seed=11, kind="gelu", x_scale=2.0)
    sp, sn, ip, ineg = oracle.calibrate_amax(x, kseg)
    wq, ws = oracle.quantize_weight(w, kseg, [24, 16], per_column)
    qp, qn = oracle.quantize_dualscale(x, kseg, ip, ineg)
    acc = oracle.segment_acc(qp, qn, wq, kseg)
    y = oracle.dequantize(acc, sp, sn, ws)
    ref = _dequant_then_matmul(qp, qn, wq, ws, sp, sn, kseg)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # the layer approximates X W: quantisation error only
    exact = fl(x).astype(np.float64) @ w.astype(np.float64)
    rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    assert rel < 0.02


def test_nonnegative_input_reduces_to_single_scale():
    """An all-nonnegative X: s- = 0, X- codes and A- vanish, and Y is the
    ordinary single-scale W8A8 product s+ s_w (q+ W_q)."""
    x, w = W.make_custom(12, 128, 32, seed=13, kind="pos")
    sp, sn, ip, ineg = oracle.calibrate_amax(x, [128])
    wq, ws = oracle.quantize_weight(w, [128], None, per_column=True)
    qp, qn = oracle.quantize_dualscale(x, [128], ip, ineg)
    acc = oracle.segment_acc(qp, qn, wq, [128])
    assert sn[0] == 0 and not qn.any() and not acc[1].any()
    y = oracle.dequantize(acc, sp, sn, ws)
    single = float(sp[0]) * (qp.astype(np.int64) @ wq.astype(np.int64)) * ws[0].astype(np.float64)
    assert np.array_equal(y, single)


def test_dualscale_beats_single_scale_on_skewed_input():
    """The point of the method [P1 DualScale motivation]: on a GELU/SiLU-like
    input (wide positive range, narrow dense negatives) two scales give a
    smaller reconstruction error of the negative values than one."""
    x, _ = W.make_custom(64, 256, 8, seed=17, kind="gelu", x_scale=3.0)
    sp, sn, ip, ineg = oracle.calibrate_amax(x, [256])
    qp, qn = oracle.quantize_dualscale(x, [256], ip, ineg)
    xf = fl(x).astype(np.float64)
    dual = float(sp[0]) * qp + float(sn[0]) * qn
    # one symmetric scale for both signs: same oracle, s- forced to s+
    s1 = float(sp[0]) if float(sp[0]) * 127 >= float(sn[0]) * 128 else float(sn[0]) * 128 / 127
    i1 = np.float32(1.0 / s1)
    qp1, qn1 = oracle.quantize_dualscale(x, [256], [i1], [i1])
    single = s1 * qp1 + s1 * qn1
    neg = xf < 0
    e_dual = np.abs(dual - xf)[neg].mean()
    e_single = np.abs(single - xf)[neg].mean()
    assert e_dual < 0.2 * e_single


# --------------------------------------------------- single-scale mode ----
@pytest.mark.parametrize("kind", ["gelu", "silu", "blocks", "neg"])
def test_single_scale_calibration(kind):
    """The single-scale baseline [P2 deployment-cost table, INT8 baseline;
    P1 limitations, DualScale per layer]: per segment the element of largest
    magnitude maps to exactly +-127, every code lies in [-127, 127], and
    negating X negates every code under the same table (one symmetric
    step, unlike the two-scale table)."""
    kseg = [64, 192]
    x, _ = W.make_custom(24, 256, 8, seed=23, kind=kind, x_scale=2.5)
    s, s2, inv, inv2 = oracle.calibrate_amax_single(x, kseg)
    assert np.array_equal(s, s2) and np.array_equal(inv, inv2)
    qp, qn = oracle.quantize_dualscale(x, kseg, inv, inv2)
    q = qp.astype(np.int32) + qn
    assert q.min() >= -127 and q.max() <= 127
    xf = fl(x)
    for i, (lo, hi) in enumerate([(0, 64), (64, 256)]):
        seg = np.abs(xf[:, lo:hi])
        r, c = np.unravel_index(np.argmax(seg), seg.shape)
        assert abs(q[r, lo + c]) == 127
    xneg = bits(-xf)
    s_n, _, inv_n, _ = oracle.calibrate_amax_single(xneg, kseg)
    assert np.array_equal(s_n, s) and np.array_equal(inv_n, inv)
    qpn, qnn = oracle.quantize_dualscale(xneg, kseg, inv_n, inv_n)
    assert np.array_equal(qpn.astype(np.int32) + qnn, -q)


def test_single_scale_nonnegative_input_matches_dualscale_positive_half():
    """On an all-nonnegative X the single range max|x| is max x, so the
    single-scale table equals the DualScale table's + half."""
    x, _ = W.make_custom(10, 128, 8, seed=29, kind="pos")
    s, _, inv, _ = oracle.calibrate_amax_single(x, [128])
    sp, _, ip, _ = oracle.calibrate_amax(x, [128])
    assert np.array_equal(s, sp) and np.array_equal(inv, ip)


@pytest.mark.parametrize("kseg", [[256], [64, 64, 128]])
def test_single_scale_layer_is_textbook_w8a8(kseg):
    """With the single-scale table, the DualScale steps compute textbook
    per-segment W8A8: codes q = clamp(rne(fp32(x * inv)), -127, 127) written
    out here with numpy fp32 arithmetic, A_i = q_i W_q,i by an int64 numpy
    matmul, y = sum_i s_i w_scale_i A_i."""
    x, w = W.make_custom(16, 256, 24, seed=31, kind="gelu", x_scale=2.0)
    s, s2, inv, inv2 = oracle.calibrate_amax_single(x, kseg)
    wq, ws = oracle.quantize_weight(w, kseg, None, per_column=True)
    qp, qn = oracle.quantize_dualscale(x, kseg, inv, inv2)
    acc = oracle.segment_acc(qp, qn, wq, kseg)
    y = oracle.dequantize(acc, s, s2, ws)
    xf = fl(x)
    edges = np.concatenate([[0], np.cumsum(kseg)])
    yt = np.zeros((16, 24))
    for i in range(len(kseg)):
        lo, hi = edges[i], edges[i + 1]
        prod = xf[:, lo:hi].astype(np.float32) * np.float32(inv[i])   # one fp32 multiply
        q = np.clip(np.rint(prod), -127, 127).astype(np.int64)         # rint: half to even
        assert np.array_equal(q, qp[:, lo:hi].astype(np.int64) + qn[:, lo:hi])
        a = q @ wq[lo:hi].astype(np.int64)
        assert np.array_equal(a, acc[0, i].astype(np.int64) + acc[1, i])
        yt += float(s[i]) * a * ws[i].astype(np.float64)
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=0)


# ------------------------------------------------ producer activations ----
@pytest.mark.parametrize("kind", ["silu", "gelu"])
def test_activation_matches_library_and_odd_part(kind):
    """[P1/P2: the SiLU/GELU producers of the asymmetric activations]
    act(0) = 0; act(z) - act(-z) = z for both (sigma(z) + sigma(-z) = 1,
    erf odd); and the values agree with torch's own fp64 functions."""
    import torch
    g = np.random.default_rng(5)
    zf = np.concatenate([g.standard_normal(4000).astype(np.float32) * 3,
                         np.array([0.0, 1.0, -1.0, 8.0, -8.0, 30.0, -30.0], np.float32)])
    z = bits(zf)
    v = oracle.activation(z, kind)
    vn = oracle.activation(bits(-fl(z)), kind)
    zz = fl(z).astype(np.float64)
    np.testing.assert_allclose(v - vn, zz, rtol=1e-14, atol=1e-300)
    assert oracle.activation(bits(np.zeros(1, np.float32)), kind)[0] == 0.0
    # torch's fp64 functions where their own evaluation is accurate (its
    # GELU goes through 1 + erf, which cancels for z below about -5)
    t = torch.from_numpy(zz)
    ref = (torch.nn.functional.silu(t) if kind == "silu" else torch.nn.functional.gelu(t)).numpy()
    ok = zz > -5.0
    np.testing.assert_allclose(v[ok], ref[ok], rtol=1e-9, atol=1e-300)
    pos = zz >= 0
    np.testing.assert_allclose(v[pos], ref[pos], rtol=1e-14, atol=1e-300)
    if kind == "gelu":
        # far left tail: GELU(z) = -phi(z) (1 - z^-2 + 3 z^-4 - 15 z^-6 + ...),
        # phi the standard normal density (asymptotic series of erfc)
        zt = np.array([-12.0, -20.0, -30.0], np.float32)
        vt = oracle.activation(bits(zt), kind)
        zz = zt.astype(np.float64)
        phi = np.exp(-zz * zz / 2) / math.sqrt(2 * math.pi)
        series = -phi * (1 - zz ** -2 + 3 * zz ** -4 - 15 * zz ** -6 + 105 * zz ** -8)
        np.testing.assert_allclose(vt, series, rtol=1e-6)


# ---------------------------------------------------- 4-bit weights (W4A8) ----
def test_w4_weight_worked_example_and_ties():
    """4-bit weights [P2 deployment-cost table, SegQuant-4; P1 W4A8]: one
    group with amax 3.5 -> s_w = 0.5, inv_w = 2 (both exact).  Worked out by
    hand: w = 3.5 -> 7; 1.25 -> 2.5 -> 2 (tie to even); 0.75 -> 1.5 -> 2;
    -0.25 -> -0.5 -> -0 = 0 (tie to even); -1.75 -> -3.5 -> -4; -3.5 -> -7."""
    w = np.array([[3.5], [1.25], [0.75], [-0.25], [-1.75], [-3.5]] + [[0.0]] * 58, np.float32)
    wq, ws = oracle.quantize_weight(w, [64], None, True, bits=4)
    assert ws[0, 0] == np.float32(0.5)
    assert wq[:6, 0].tolist() == [7, 2, 2, 0, -4, -7]
    assert not wq[6:].any()


@pytest.mark.parametrize("per_column", [False, True])
def test_w4_weight_groups_range_and_error(per_column):
    """Codes in [-7, 7]; the largest |w| of each group maps to +-7; every
    element within half a step of its reconstruction (up to the fp32
    rounding of the product); groups as for int8 weights."""
    g = np.random.default_rng(3)
    K, N, kseg, nseg = 192, 48, [64, 128], [16, 32]
    w = (g.standard_normal((K, N)) * np.repeat([0.02, 0.3], [16, 32])[None, :]).astype(np.float32)
    wq, ws = oracle.quantize_weight(w, kseg, None if per_column else nseg, per_column, bits=4)
    assert wq.min() >= -7 and wq.max() <= 7
    w8, ws8 = oracle.quantize_weight(w, kseg, None if per_column else nseg, per_column, bits=8)
    # same groups: the 4-bit step is the int8 step times 127/7 (each rounded once)
    np.testing.assert_allclose(ws.astype(np.float64), ws8.astype(np.float64) * 127 / 7, rtol=2e-7)
    rec = wq.astype(np.float64) * np.repeat(ws, kseg, axis=0)
    step = np.repeat(ws, kseg, axis=0).astype(np.float64)
    assert np.all(np.abs(rec - w) <= 0.5 * step * (1 + 1e-6) + 1e-12)
    for i, (lo, hi) in enumerate([(0, 64), (64, 192)]):
        groups = [(c, c + 1) for c in range(N)] if per_column else [(0, 16), (16, 48)]
        for c0, c1 in groups:
            blk = np.abs(w[lo:hi, c0:c1])
            r, c = np.unravel_index(np.argmax(blk), blk.shape)
            assert abs(int(wq[lo + r, c0 + c])) == 7


def test_composed_linear_equals_steps():
    x, w = W.make_custom(23, 256, 48, seed=19, kind="blocks")
    kseg = [64, 64, 128]
    sp, sn, ip, ineg = oracle.calibrate_amax(x, kseg)
    wq, ws = oracle.quantize_weight(w, kseg, None, per_column=False)
    qp, qn = oracle.quantize_dualscale(x, kseg, ip, ineg)
    y1 = oracle.dequantize(oracle.segment_acc(qp, qn, wq, kseg), sp, sn, ws)
    y2 = oracle.dualscale_linear(x, wq, ws, kseg, sp, sn, ip, ineg)
    assert np.array_equal(y1, y2)


# ------------------------------------------------------------ generators ----
def test_adanorm_generator_matches_printed_polarity():
    """The AdaNorm workload's share of negative-dominant channels matches the
    printed AdaNorm(DiT) row of the polarity table (golden fixture)."""
    path = os.path.join(os.path.dirname(__file__), "golden", "polarity_table.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    neg_frac = {r[0]: float(r[3]) for r in rows}["AdaNorm(DiT)"]
    wl, x, _ = W.make_inputs("c2_adanorm_gemv")
    xf = fl(x)
    # a channel is negative-dominant when at least half of its values are < 0
    frac = float(((xf < 0).mean(axis=0) >= 0.5).mean())
    assert abs(frac - neg_frac) < 0.03
    assert xf.min() > -0.3 and xf.max() < 4.0  # SiLU range, cf. the stated ranges


def test_workload_shapes():
    for name in ("c1_tiny_outseg", "c2_adanorm_gemv", "c4_attn_out_inseg"):
        wl, x, w = W.make_inputs(name)
        assert x.shape == (wl.M, wl.K) and x.dtype == np.uint16
        assert w.shape == (wl.K, wl.N) and w.dtype == np.float32
        assert sum(wl.kseg) == wl.K and sum(wl.nseg) == wl.N
        assert all(s % 64 == 0 for s in wl.kseg)
    assert W.WORKLOADS["c5_flux_ffn_fc2"].M * W.WORKLOADS["c5_flux_ffn_fc2"].K == 113246208
