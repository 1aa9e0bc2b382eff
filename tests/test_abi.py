"""The C ABI without a GPU: the library loads, exports every function that
include/segquant.h declares, and rejects invalid arguments with the
documented status before any HIP call (so nothing is enqueued)."""
import ctypes
import os
import re
import threading

import numpy as np
import pytest

import segmented_dual_scale_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "segquant.h")


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# The calls below pass fake (non-NULL, aligned) device addresses; each is
# built to fail validation, which happens before any HIP call.  On a machine
# with a GPU a validation bug could turn one into a launch on a bogus
# address, so this module runs on CPU-only machines.
pytestmark = pytest.mark.skipif(_gpu_present(), reason="fake device pointers: CPU-only tests")

FAKE = ctypes.c_void_p(0x10000)
P = ctypes.c_void_p


def lib():
    return S.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(segquant_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    so = ctypes.CDLL(S.library_path())
    for n in names:
        assert hasattr(so, n), n


def test_version_and_status_strings():
    assert S.segquant_version() >= 100
    codes = [S.SEGQ_OK, S.SEGQ_ERR_NULL, S.SEGQ_ERR_SHAPE, S.SEGQ_ERR_SEGMENTS, S.SEGQ_ERR_ALIGN,
             S.SEGQ_ERR_UNSUPPORTED, S.SEGQ_ERR_HIP]
    texts = [S.segquant_status_string(c) for c in codes]
    assert len(set(texts)) == len(codes)
    assert S.segquant_status_string(12345) == "unknown status"


def test_packed_bytes():
    assert S.segquant_weight_packed_bytes(1536, 9216) == 1536 * 9216
    assert S.segquant_weight_packed_bytes(100, 16) == 0
    assert S.segquant_weight_packed_bytes(64, 10) == 0
    assert S.segquant_weight_packed_bytes(0, 16) == 0


def test_gemm_halves_from_host_scales():
    """One product per element only when no K-segment has a negative half."""
    a = np.zeros((4, 3), np.float32)
    a[0] = [0.1, 0.2, 0.3]
    a[2] = 1.0 / a[0]
    assert S.segquant_gemm_halves(a) == S.SEGQ_GEMM_SINGLE_SCALE
    b = a.copy()
    b[1, 2], b[3, 2] = 0.01, 100.0  # the last segment has negative values
    assert S.segquant_gemm_halves(b) == 0
    c = a.copy()
    c[3, 1] = 5.0  # an inverse without its scale still quantises a - half
    assert S.segquant_gemm_halves(c) == 0
    assert lib().segquant_gemm_halves(None, 3) == S.SEGQ_ERR_NULL
    assert lib().segquant_gemm_halves(a.ctypes.data, 0) == S.SEGQ_ERR_SEGMENTS
    big = np.zeros((4, 129), np.float32)
    assert lib().segquant_gemm_halves(big.ctypes.data, 129) == S.SEGQ_ERR_SEGMENTS
    with pytest.raises(ValueError):
        S.segquant_gemm_halves(np.zeros((3, 2), np.float32))


def test_kernel_choice():
    assert S.segquant_gemm_kernel_for(2, 9216, 1536) == S.SEGQ_KERNEL_SMALLM
    assert S.segquant_gemm_kernel_for(16, 64, 64) == S.SEGQ_KERNEL_SMALLM
    assert S.segquant_gemm_kernel_for(17, 64, 64) == S.SEGQ_KERNEL_TILE
    assert S.segquant_gemm_kernel_for(2, 64, 64, S.SEGQ_GEMM_FORCE_TILE) == S.SEGQ_KERNEL_TILE
    assert S.segquant_gemm_kernel_for(17, 64, 64, S.SEGQ_GEMM_FORCE_SMALLM) == S.SEGQ_ERR_UNSUPPORTED
    assert S.segquant_gemm_kernel_for(64, 64, 100) == S.SEGQ_ERR_ALIGN


def segs(widths):
    w = np.asarray(widths, np.int32)
    off = np.zeros_like(w)
    if len(w) > 1:
        off[1:] = np.cumsum(w)[:-1]
    return off, w


def gemm(M=64, N=64, K=128, x=FAKE, ld_x=None, xq=None, ld_q=0, q_layout=0, w=FAKE, ws=FAKE,
         widths=None, off=None, act=FAKE, y=FAKE, ld_y=None, acc=None, flags=0, n_kseg=None,
         work=None, work_bytes=0, noalloc=False):
    o, wd = segs(widths if widths is not None else [K])
    if off is not None:
        o = np.asarray(off, np.int32)
    args = (M, N, K, x, K if ld_x is None else ld_x, xq, ld_q, q_layout, w, ws,
            len(wd) if n_kseg is None else n_kseg, o.ctypes.data_as(P), wd.ctypes.data_as(P), act,
            y, N if ld_y is None else ld_y, acc)
    if noalloc:  # the no-allocation entry point: same arguments less the workspace
        return lib().segquant_gemm_w8a8_seg_noalloc(*args, flags, None)
    return lib().segquant_gemm_w8a8_seg(*args, work, work_bytes, flags, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(K=100), S.SEGQ_ERR_ALIGN),
    (dict(N=40), S.SEGQ_ERR_ALIGN),
    (dict(M=-1), S.SEGQ_ERR_SHAPE),
    (dict(K=0), S.SEGQ_ERR_SHAPE),
    (dict(M=1 << 40), S.SEGQ_ERR_SHAPE),
    (dict(x=None), S.SEGQ_ERR_NULL),
    (dict(xq=FAKE, ld_q=128), S.SEGQ_ERR_NULL),
    (dict(ld_x=120), S.SEGQ_ERR_SHAPE),
    (dict(ld_x=132), S.SEGQ_ERR_ALIGN),
    (dict(x=ctypes.c_void_p(0x10008)), S.SEGQ_ERR_ALIGN),
    (dict(x=None, xq=FAKE, ld_q=136), S.SEGQ_ERR_ALIGN),
    (dict(x=None, xq=FAKE, ld_q=64), S.SEGQ_ERR_SHAPE),
    (dict(x=None, xq=FAKE, ld_q=128, q_layout=7), S.SEGQ_ERR_SHAPE),
    (dict(x=None, xq=ctypes.c_void_p(0x10004), ld_q=128), S.SEGQ_ERR_ALIGN),
    (dict(w=None), S.SEGQ_ERR_NULL),
    (dict(ws=None), S.SEGQ_ERR_NULL),
    (dict(act=None), S.SEGQ_ERR_NULL),
    (dict(y=None), S.SEGQ_ERR_NULL),
    (dict(w=ctypes.c_void_p(0x10001)), S.SEGQ_ERR_ALIGN),
    (dict(y=ctypes.c_void_p(0x10001)), S.SEGQ_ERR_ALIGN),
    (dict(acc=ctypes.c_void_p(0x10002)), S.SEGQ_ERR_ALIGN),
    (dict(ld_y=48), S.SEGQ_ERR_SHAPE),
    (dict(widths=[64]), S.SEGQ_ERR_SEGMENTS),                # does not cover K
    (dict(widths=[64, 64], off=[0, 32]), S.SEGQ_ERR_SEGMENTS),  # not contiguous
    (dict(widths=[128, 0]), S.SEGQ_ERR_SEGMENTS),
    (dict(widths=[96, 32]), S.SEGQ_ERR_ALIGN),               # boundary not on 64
    (dict(widths=[128], n_kseg=0), S.SEGQ_ERR_SEGMENTS),
    (dict(K=64 * 129, widths=[64] * 129), S.SEGQ_ERR_UNSUPPORTED),
    (dict(K=132160, widths=[132160]), S.SEGQ_ERR_UNSUPPORTED),  # int32 bound
    (dict(M=17, flags=S.SEGQ_GEMM_FORCE_SMALLM), S.SEGQ_ERR_UNSUPPORTED),
    (dict(flags=3), S.SEGQ_ERR_SHAPE),
    (dict(flags=32), S.SEGQ_ERR_SHAPE),
    (dict(x=None, xq=FAKE, ld_q=128, q_layout=1, flags=8), S.SEGQ_ERR_UNSUPPORTED),
])
@pytest.mark.parametrize("noalloc", [False, True])
def test_gemm_validation(kwargs, status, noalloc):
    assert gemm(noalloc=noalloc, **kwargs) == status
    assert S.segquant_last_error() != ""


def test_noalloc_refuses_a_widening_beyond_its_scratch():
    """4-bit weights off the streaming kernel are widened to K*N int8 bytes;
    beyond the no-allocation call's scratch that is refused before any HIP
    call (a quantise-first workspace beyond it is not needed: the call then
    quantises inside the GEMM)."""
    K, N = 8192, 16384  # 128 MiB widened
    assert K * N > S.SEGQ_NOALLOC_SCRATCH_BYTES
    assert gemm(M=64, N=N, K=K, flags=S.SEGQ_GEMM_W4, noalloc=True) == S.SEGQ_ERR_UNSUPPORTED
    assert "scratch" in S.segquant_last_error()


def test_gemm_w4_needs_a_workspace_off_the_streaming_kernel():
    """4-bit weights on a large-M shape are widened in the workspace first:
    without one (or with too small a one) the call fails before any launch."""
    assert gemm(M=64, flags=S.SEGQ_GEMM_W4) == S.SEGQ_ERR_UNSUPPORTED
    assert "workspace" in S.segquant_last_error()
    assert gemm(M=64, flags=S.SEGQ_GEMM_W4, work=FAKE, work_bytes=64 * 128 - 16) == S.SEGQ_ERR_UNSUPPORTED
    assert S.segquant_gemm_workspace_bytes(64, 64, 128, None, S.SEGQ_GEMM_W4) == 64 * 128
    # the streaming small-M kernel reads the 4-bit tiles itself
    assert S.segquant_gemm_workspace_bytes(2, 9216, 1536, None, S.SEGQ_GEMM_W4) == 0
    assert S.segquant_weight_packed_bytes(1536, 9216) == 2 * S.load_library().segquant_weight_packed_bytes_w4(1536, 9216)


def test_gemm_accepts_several_segments_beyond_the_int32_bound_of_k():
    """Only each K-segment's width is bounded (its int32 sums); a K above that
    bound split into narrower segments passes validation (and asks for no
    workspace: the segments are folded inside the GEMM)."""
    K = 132160
    assert S.segquant_gemm_workspace_bytes(40, 64, K, [66048, 66112]) == 0
    assert S.segquant_last_error() == ""
    assert S.segquant_gemm_workspace_bytes(40, 64, K, [K]) == 0
    assert "int32 bound" in S.segquant_last_error()


def test_gemm_misaligned_workspace():
    assert gemm(work=ctypes.c_void_p(0x10008), work_bytes=1 << 20) == S.SEGQ_ERR_ALIGN
    assert "workspace" in S.segquant_last_error()


@pytest.mark.parametrize("M,N,K,widths,flags,expect", [
    (4096, 1536, 6144, None, 0, 0),                        # one segment: tiles of 384, 4 across
    (4429, 1536, 1536, [64] * 24, 0, 4429 * 1536),         # tiles of 256, 6 across
    (9216, 3072, 12288, [3072] * 4, 0, 9216 * 12288),      # 12 across
    (9216, 3072, 12288, [3072] * 4, S.SEGQ_GEMM_FUSED_QUANT, 0),
    (300, 2304, 512, None, 0, 300 * 512),                  # one segment, 6 tiles of 384
    (300, 1920, 512, None, 0, 0),                          # 5 tiles
    (16, 9216, 1536, None, 0, 0),                          # small M: the streaming kernel
    (64, 9216, 1536, None, S.SEGQ_GEMM_FORCE_SMALLM, None),  # invalid: forced small-M, M > 16
])
def test_gemm_workspace_bytes(M, N, K, widths, flags, expect):
    got = S.segquant_gemm_workspace_bytes(M, N, K, widths, flags)
    if expect is None:
        assert got == 0 and S.segquant_last_error() != ""
    else:
        assert got == expect and S.segquant_last_error() == ""


def test_gemm_null_segment_arrays():
    rc = lib().segquant_gemm_w8a8_seg(64, 64, 128, FAKE, 128, None, 0, 0, FAKE, FAKE, 1, None,
                                      None, FAKE, FAKE, 64, None, None, 0, 0, None)
    assert rc == S.SEGQ_ERR_NULL


def test_empty_batch_is_ok_without_launch():
    assert gemm(M=0, x=None, y=None) == S.SEGQ_OK
    assert S.segquant_last_error() == ""


def test_last_error_is_thread_local():
    assert gemm(K=100) == S.SEGQ_ERR_ALIGN
    seen = {}

    def other():
        seen["before"] = S.segquant_last_error()
        gemm(N=40)
        seen["after"] = S.segquant_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["before"] == ""
    assert "N=40" in seen["after"]
    assert "K=100" in S.segquant_last_error()


def quant(M=8, K=128, x=FAKE, ld_x=None, widths=None, act=FAKE, q=FAKE, ld_q=128, layout=0):
    o, wd = segs(widths if widths is not None else [K])
    return lib().segquant_quantize_dualscale(x, M, K, K if ld_x is None else ld_x, len(wd),
                                             o.ctypes.data_as(P), wd.ctypes.data_as(P), act, q,
                                             ld_q, layout, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), S.SEGQ_ERR_NULL),
    (dict(act=None), S.SEGQ_ERR_NULL),
    (dict(q=None), S.SEGQ_ERR_NULL),
    (dict(layout=2), S.SEGQ_ERR_SHAPE),
    (dict(ld_q=112), S.SEGQ_ERR_SHAPE),
    (dict(ld_q=136), S.SEGQ_ERR_ALIGN),
    (dict(q=ctypes.c_void_p(0x10008)), S.SEGQ_ERR_ALIGN),
    (dict(ld_x=100), S.SEGQ_ERR_SHAPE),
    (dict(K=130, ld_x=130, ld_q=144, widths=[130]), S.SEGQ_ERR_ALIGN),  # ld_x % 8
    (dict(widths=[32, 96]), S.SEGQ_ERR_ALIGN),
    (dict(widths=[64]), S.SEGQ_ERR_SEGMENTS),
    (dict(M=-3), S.SEGQ_ERR_SHAPE),
])
def test_quantize_validation(kwargs, status):
    assert quant(**kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), S.SEGQ_ERR_NULL),
    (dict(act=None), S.SEGQ_ERR_NULL),
    (dict(widths=[64, 65]), S.SEGQ_ERR_SEGMENTS),
    (dict(ld_x=64), S.SEGQ_ERR_SHAPE),
])
def test_calibrate_validation(kwargs, status):
    K = 128
    o, wd = segs(kwargs.get("widths", [K]))
    rc = lib().segquant_calibrate_amax(kwargs.get("x", FAKE), 8, K, kwargs.get("ld_x", K), len(wd),
                                       o.ctypes.data_as(P), wd.ctypes.data_as(P),
                                       kwargs.get("act", FAKE), None)
    assert rc == status


@pytest.mark.parametrize("K,N,ld_w,kw,nw,per_column,ptrs,status", [
    (100, 16, 16, [100], [16], 0, (FAKE, FAKE, FAKE), S.SEGQ_ERR_ALIGN),
    (64, 24, 24, [64], [24], 0, (FAKE, FAKE, FAKE), S.SEGQ_ERR_ALIGN),
    (64, 16, 8, [64], [16], 0, (FAKE, FAKE, FAKE), S.SEGQ_ERR_SHAPE),
    (64, 16, 16, [64], [16], 0, (None, FAKE, FAKE), S.SEGQ_ERR_NULL),
    (64, 16, 16, [64], [16], 0, (FAKE, None, FAKE), S.SEGQ_ERR_NULL),
    (64, 16, 16, [64], [16], 0, (FAKE, FAKE, None), S.SEGQ_ERR_NULL),
    (64, 16, 16, [64], [16], 0, (FAKE, ctypes.c_void_p(0x10004), FAKE), S.SEGQ_ERR_ALIGN),
    (64, 32, 32, [64], [16, 8], 0, (FAKE, FAKE, FAKE), S.SEGQ_ERR_SEGMENTS),
    (128, 16, 16, [64], [16], 0, (FAKE, FAKE, FAKE), S.SEGQ_ERR_SEGMENTS),
    (128, 16, 16, [64, 32], [16], 0, (FAKE, FAKE, FAKE), S.SEGQ_ERR_ALIGN),
])
def test_weight_validation(K, N, ld_w, kw, nw, per_column, ptrs, status):
    ko, kwd = segs(kw)
    no, nwd = segs(nw)
    rc = lib().segquant_quantize_weight(ptrs[0], K, N, ld_w, len(kwd), ko.ctypes.data_as(P),
                                        kwd.ctypes.data_as(P), len(nwd), no.ctypes.data_as(P),
                                        nwd.ctypes.data_as(P), per_column, ptrs[1], ptrs[2], None)
    assert rc == status


def test_unpack_validation():
    assert lib().segquant_unpack_weight(FAKE, 100, 16, FAKE, 16, None) == S.SEGQ_ERR_ALIGN
    assert lib().segquant_unpack_weight(FAKE, 64, 16, FAKE, 8, None) == S.SEGQ_ERR_SHAPE
    assert lib().segquant_unpack_weight(None, 64, 16, FAKE, 16, None) == S.SEGQ_ERR_NULL


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(S, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(S, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        S.load_library()
