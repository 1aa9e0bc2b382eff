"""The no-allocation entry point (segquant_gemm_w8a8_seg_noalloc) against the
ordinary one (segquant_gemm_w8a8_seg with a workspace from torch), through
the C ABI: per-segment int32 accumulators and bf16 Y bit-identical, on two
calls in a row with the second on a smaller input (the shared scratch keeps
the first call's contents).  Cases that use the scratch: quantise-first
codes (24 K-segments, six column tiles) and the int8 widening of 4-bit
weights on the large-M kernel; and a quantise-first call too large for the
scratch, which runs the fused launch instead."""
import numpy as np
import pytest

import segmented_dual_scale_amd as S
from segmented_dual_scale_amd import workloads as W
from gpu_common import DEV, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _layer(M, K, N, kseg, bits, seed):
    import torch
    x, w = W.make_custom(M, K, N, seed=seed, kind="blocks", x_scale=2.0)
    xd = to_dev_bf16(x)
    act = S.segquant_calibrate_amax(xd, kseg)
    wp, ws = S.segquant_quantize_weight(to_dev(w), kseg, None, True, bits=bits)
    torch.cuda.synchronize()
    return xd, act, wp, ws


def _both(M, K, N, kseg, bits, seed):
    import torch
    xd, act, wp, ws = _layer(M, K, N, kseg, bits, seed)
    flags = S.SEGQ_GEMM_W4 if bits == 4 else S.SEGQ_GEMM_AUTO
    nb = S.segquant_gemm_workspace_bytes(M, N, K, kseg, flags)
    assert nb > 0, "the case must use the workspace"
    acc_a = torch.full((2, len(kseg), M, N), -7, dtype=torch.int32, device=DEV)
    y_a = S.segquant_gemm_w8a8_seg(xd, wp, ws, act, kseg, acc_debug=acc_a, workspace="auto",
                                   flags=flags)
    acc_b = torch.full((2, len(kseg), M, N), -9, dtype=torch.int32, device=DEV)
    y_b = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    S.segquant_gemm_w8a8_seg_noalloc(xd, wp, ws, act, y_b, kseg, acc_debug=acc_b, flags=flags)
    y_c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    S.segquant_gemm_w8a8_seg_noalloc(xd, wp, ws, act, y_c, kseg, flags=flags)  # timed form
    torch.cuda.synchronize()
    assert torch.equal(acc_a, acc_b), "per-segment accumulators differ"
    assert torch.equal(y_a.view(torch.int16), y_b.view(torch.int16)), "Y differs (debug form)"
    assert torch.equal(y_a.view(torch.int16), y_c.view(torch.int16)), "Y differs"


@pytest.mark.parametrize("first,second", [
    # quantise-first codes in the scratch: 24 K-segments of 64, six tiles of 256 columns
    ((300, 1536, 1536, [64] * 24, 8), (100, 768, 1536, [64] * 12, 8)),
    # 4-bit weights widened to int8 tiles in the scratch, large-M kernel
    ((77, 512, 768, [256, 256], 4), (33, 256, 512, [256], 4)),
])
def test_noalloc_matches_the_workspace_call_twice(first, second):
    M, K, N, kseg, bits = first
    _both(M, K, N, kseg, bits, seed=1)
    M, K, N, kseg, bits = second
    _both(M, K, N, kseg, bits, seed=2)


def test_noalloc_runs_fused_when_codes_exceed_the_scratch():
    """M*K codes above the scratch: the no-allocation call quantises inside
    the GEMM (SEGQ_GEMM_FUSED_QUANT), bit-identical to that fused call."""
    import torch
    M, K, N, kseg = 4480, 15360, 1536, [3840] * 4
    assert M * K > S.SEGQ_NOALLOC_SCRATCH_BYTES
    assert S.segquant_gemm_workspace_bytes(M, N, K, kseg) == M * K
    xd, act, wp, ws = _layer(M, K, N, kseg, 8, seed=3)
    y_f = S.segquant_gemm_w8a8_seg(xd, wp, ws, act, kseg, workspace=None,
                                   flags=S.SEGQ_GEMM_FUSED_QUANT)
    y_n = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    S.segquant_gemm_w8a8_seg_noalloc(xd, wp, ws, act, y_n, kseg)
    torch.cuda.synchronize()
    assert torch.equal(y_f.view(torch.int16), y_n.view(torch.int16))
