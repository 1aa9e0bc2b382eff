"""segmented_dual_scale_amd -- SegQuant's DualScale x SegLinear W8A8 linear
layer on AMD Instinct MI355X (gfx950).

This module is a thin ctypes binding over the C ABI of ``libsegquant.so``
(``include/segquant.h``).  Each function has the name of its C entry point and
only marshals arguments: torch supplies device memory and the current HIP
stream, every step of the layer runs in the library's HIP kernels.  If the
library is not built, every call raises: there is no other path.

    from segmented_dual_scale_amd import (segquant_calibrate_amax,
        segquant_quantize_weight, segquant_gemm_w8a8_seg)
    act = segquant_calibrate_amax(x, kseg=[64] * 24)            # offline
    wq, ws = segquant_quantize_weight(w, kseg=[64] * 24)        # offline
    y = segquant_gemm_w8a8_seg(x, wq, ws, act, kseg=[64] * 24)  # one launch

Pages: "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
for Diffusion Models" (papernotes.org notes, "SegLinear" and "DualScale"
sections) and "SegQuant" (hliangzhao.me, sections 2 and 3).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

__all__ = [
    "SegQuantError", "library_path", "load_library",
    "segquant_calibrate_amax", "segquant_quantize_dualscale", "segquant_weight_packed_bytes",
    "segquant_quantize_weight", "segquant_unpack_weight", "segquant_gemm_w8a8_seg",
    "segquant_gemm_kernel_for", "segquant_status_string", "segquant_last_error",
    "segquant_version", "SEGQ_Q_SIGNED", "SEGQ_Q_PLANES", "SEGQ_GEMM_AUTO",
    "SEGQ_GEMM_FORCE_TILE", "SEGQ_GEMM_FORCE_SMALLM", "SEGQ_GEMM_FUSED_QUANT",
    "SEGQ_GEMM_SINGLE_SCALE", "segquant_calibrate_amax_single",
    "SEGQ_ACT_SILU", "SEGQ_ACT_GELU", "segquant_activate_quantize", "SEGQ_GEMM_W4", "SEGQ_KERNEL_TILE", "SEGQ_KERNEL_SMALLM",
    "segquant_gemm_halves", "segquant_gemm_w8a8_seg_noalloc", "SEGQ_NOALLOC_SCRATCH_BYTES",
]

SEGQ_OK = 0
SEGQ_ERR_NULL = -1
SEGQ_ERR_SHAPE = -2
SEGQ_ERR_SEGMENTS = -3
SEGQ_ERR_ALIGN = -4
SEGQ_ERR_UNSUPPORTED = -5
SEGQ_ERR_HIP = -6
SEGQ_MAX_KSEG = 128
SEGQ_MAX_KSEG_WIDTH = 132104
SEGQ_Q_SIGNED = 0
SEGQ_Q_PLANES = 1
SEGQ_GEMM_AUTO = 0
SEGQ_GEMM_FORCE_TILE = 1
SEGQ_GEMM_FORCE_SMALLM = 2
SEGQ_GEMM_FUSED_QUANT = 4
SEGQ_GEMM_SINGLE_SCALE = 8
SEGQ_GEMM_W4 = 16
SEGQ_ACT_SILU = 1
SEGQ_ACT_GELU = 2
SEGQ_KERNEL_TILE = 1
SEGQ_KERNEL_SMALLM = 2
SEGQ_NOALLOC_SCRATCH_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
# SEGQUANT_LIBRARY names another build of the same library (the tests use it
# for a build whose host code carries address and undefined-behaviour
# sanitizers); by default the in-tree build is loaded.
_LIB_PATH = os.environ.get("SEGQUANT_LIBRARY") or os.path.join(_HERE, "libsegquant.so")
_lib = None


class SegQuantError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({segquant_status_string(status)}): {detail}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsegquant.so (built in-tree by segmented_dual_scale_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m segmented_dual_scale_amd.build` "
                           "(the layer has no other implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    sig = {
        "segquant_calibrate_amax": [P, I64, I64, I64, I32, P, P, P, P],
        "segquant_calibrate_amax_single": [P, I64, I64, I64, I32, P, P, P, P],
        "segquant_activate_quantize": [P, I64, I64, I64, I32, I32, P, P, P, P, I64, I32, P, I64,
                                       P],
        "segquant_quantize_dualscale": [P, I64, I64, I64, I32, P, P, P, P, I64, I32, P],
        "segquant_quantize_weight": [P, I64, I64, I64, I32, P, P, I32, P, P, I32, P, P, P],
        "segquant_unpack_weight": [P, I64, I64, P, I64, P],
        "segquant_unpack_weight_w4": [P, I64, I64, P, I64, P],
        "segquant_quantize_weight_w4": [P, I64, I64, I64, I32, P, P, I32, P, P, I32, P, P, P],
        "segquant_weight_packed_bytes_w4": [I64, I64],
        "segquant_gemm_w8a8_seg": [I64, I64, I64, P, I64, P, I64, I32, P, P, I32, P, P, P, P, I64,
                                   P, P, ctypes.c_size_t, U32, P],
        "segquant_gemm_w8a8_seg_noalloc": [I64, I64, I64, P, I64, P, I64, I32, P, P, I32, P, P,
                                           P, P, I64, P, U32, P],
        "segquant_gemm_workspace_bytes": [I64, I64, I64, I32, P, P, U32],
        "segquant_gemm_kernel_for": [I64, I64, I64, U32],
        "segquant_gemm_halves": [P, I32],
        "segquant_version": [],
        "segquant_status_string": [ctypes.c_int],
        "segquant_last_error": [],
        "segquant_weight_packed_bytes": [I64, I64],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.segquant_status_string.restype = ctypes.c_char_p
    lib.segquant_last_error.restype = ctypes.c_char_p
    lib.segquant_weight_packed_bytes.restype = ctypes.c_size_t
    lib.segquant_weight_packed_bytes_w4.restype = ctypes.c_size_t
    lib.segquant_gemm_workspace_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


# ----------------------------------------------------------------- helpers --
def _segs(widths: Optional[Sequence[int]], total: int):
    import numpy as np
    w = np.asarray(list(widths) if widths is not None else [total], dtype=np.int32)
    off = np.zeros_like(w)
    if len(w) > 1:
        off[1:] = np.cumsum(w)[:-1]
    return off, w


def _arr_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(rc: int, where: str):
    if rc != SEGQ_OK:
        raise SegQuantError(rc, where, segquant_last_error())


def _ld(t, what: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{what} must be a 2-D tensor with unit stride in its last dimension")
    return t.stride(0)


# --------------------------------------------------------------- the ABI ----
def segquant_status_string(status: int) -> str:
    return load_library().segquant_status_string(status).decode()


def segquant_last_error() -> str:
    return load_library().segquant_last_error().decode()


def segquant_version() -> int:
    return load_library().segquant_version()


def segquant_weight_packed_bytes(K: int, N: int) -> int:
    return int(load_library().segquant_weight_packed_bytes(K, N))


def segquant_gemm_kernel_for(M: int, N: int, K: int, flags: int = SEGQ_GEMM_AUTO) -> int:
    return int(load_library().segquant_gemm_kernel_for(M, N, K, flags))


def segquant_gemm_halves(act) -> int:
    """SEGQ_GEMM_SINGLE_SCALE when the scale table `act` ([4][n_kseg], device
    or host tensor, or a numpy array) has no negative half, else 0.  A device
    table is copied to the host (once per layer: the scales are static)."""
    import numpy as np
    if hasattr(act, "detach"):
        act = act.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(act, dtype=np.float32))
    if a.ndim != 2 or a.shape[0] != 4:
        raise ValueError(f"scale table of shape {a.shape}, expected [4][n_kseg]")
    r = load_library().segquant_gemm_halves(a.ctypes.data, a.shape[1])
    if r < 0:
        raise SegQuantError(r, "segquant_gemm_halves", segquant_last_error())
    return int(r)


def _calibrate(fn, name, x, kseg, out):
    import torch
    M, K = x.shape
    off, wid = _segs(kseg, K)
    if out is None:
        out = torch.empty((4, len(wid)), dtype=torch.float32, device=x.device)
    _check(fn(_ptr(x), M, K, _ld(x, "x"), len(wid), _arr_ptr(off), _arr_ptr(wid), _ptr(out),
              _stream(x)), name)
    return out


def segquant_calibrate_amax(x, kseg: Optional[Sequence[int]] = None, out=None):
    """AMax calibration: returns the fp32 [4][n_kseg] table (s+, s-, inv+,
    inv-) for bf16 X [M][K] (device)."""
    return _calibrate(load_library().segquant_calibrate_amax, "segquant_calibrate_amax", x, kseg,
                      out)


def segquant_calibrate_amax_single(x, kseg: Optional[Sequence[int]] = None, out=None):
    """Single-scale calibration: the same table layout with s+ = s- =
    max|x|/127 and inv+ = inv- = 127/max|x| per K-segment (use with
    SEGQ_GEMM_SINGLE_SCALE)."""
    return _calibrate(load_library().segquant_calibrate_amax_single,
                      "segquant_calibrate_amax_single", x, kseg, out)


def segquant_quantize_dualscale(x, act_scales, kseg: Optional[Sequence[int]] = None,
                                layout: int = SEGQ_Q_SIGNED, out=None):
    """Polarity split + dual-scale quantisation of bf16 X -> int8: [M][K]
    signed codes, or [2][M][K] planes (q+, q-)."""
    import torch
    lib = load_library()
    M, K = x.shape
    off, wid = _segs(kseg, K)
    if out is None:
        ldq = (K + 15) // 16 * 16
        shape = (M, ldq) if layout == SEGQ_Q_SIGNED else (2, M, ldq)
        out = torch.empty(shape, dtype=torch.int8, device=x.device)
    ld_q = out.stride(-2)
    _check(lib.segquant_quantize_dualscale(_ptr(x), M, K, _ld(x, "x"), len(wid), _arr_ptr(off),
                                           _arr_ptr(wid), _ptr(act_scales), _ptr(out), ld_q,
                                           layout, _stream(x)),
           "segquant_quantize_dualscale")
    return out


def segquant_activate_quantize(z, act_kind: int, act_scales=None,
                               kseg: Optional[Sequence[int]] = None,
                               layout: int = SEGQ_Q_SIGNED, out=None, x_out=None,
                               want_codes: bool = True):
    """SiLU/GELU of bf16 pre-activation Z fused with the dual-scale
    quantisation.  Returns (codes or None, x_out or None): codes as
    segquant_quantize_dualscale (when act_scales is given and want_codes),
    x_out the bf16 activation if a tensor is passed (or x_out=True to
    allocate one)."""
    import torch
    lib = load_library()
    M, K = z.shape
    off, wid = _segs(kseg, K)
    if want_codes and act_scales is not None and out is None:
        ldq = (K + 15) // 16 * 16
        shape = (M, ldq) if layout == SEGQ_Q_SIGNED else (2, M, ldq)
        out = torch.empty(shape, dtype=torch.int8, device=z.device)
    if not (want_codes and act_scales is not None):
        out = None
    if x_out is True:
        x_out = torch.empty((M, K), dtype=torch.bfloat16, device=z.device)
    ld_q = out.stride(-2) if out is not None else 0
    ld_xo = _ld(x_out, "x_out") if x_out is not None else 0
    _check(lib.segquant_activate_quantize(_ptr(z), M, K, _ld(z, "z"), act_kind, len(wid),
                                          _arr_ptr(off), _arr_ptr(wid), _ptr(act_scales), _ptr(out),
                                          ld_q, layout, _ptr(x_out), ld_xo, _stream(z)),
           "segquant_activate_quantize")
    return out, x_out


def segquant_quantize_weight(w, kseg: Optional[Sequence[int]] = None,
                             nseg: Optional[Sequence[int]] = None, per_column: bool = False,
                             out_packed=None, out_scale=None, bits: int = 8) -> Tuple:
    """Per-group symmetric int8 (bits=8) or 4-bit (bits=4, W4A8) quantisation
    of fp32 W [K][N] (device): returns (packed weight, fp32 w_scale
    [n_kseg][N])."""
    import torch
    lib = load_library()
    if bits not in (4, 8):
        raise ValueError("bits must be 8 or 4")
    K, N = w.shape
    koff, kwid = _segs(kseg, K)
    noff, nwid = _segs(nseg, N)
    if out_packed is None:
        nbytes = (segquant_weight_packed_bytes(K, N) if bits == 8
                  else int(lib.segquant_weight_packed_bytes_w4(K, N)))
        out_packed = torch.empty(max(nbytes, 16), dtype=torch.int8, device=w.device)
    if out_scale is None:
        out_scale = torch.empty((len(kwid), N), dtype=torch.float32, device=w.device)
    fn = lib.segquant_quantize_weight if bits == 8 else lib.segquant_quantize_weight_w4
    _check(fn(_ptr(w), K, N, _ld(w, "w"), len(kwid), _arr_ptr(koff), _arr_ptr(kwid), len(nwid),
              _arr_ptr(noff), _arr_ptr(nwid), int(bool(per_column)), _ptr(out_packed),
              _ptr(out_scale), _stream(w)),
           "segquant_quantize_weight" + ("" if bits == 8 else "_w4"))
    return out_packed, out_scale


def segquant_unpack_weight(w_packed, K: int, N: int, out=None, bits: int = 8):
    """Packed weight (int8, or 4-bit with bits=4) -> int8 W_q [K][N]."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty((K, N), dtype=torch.int8, device=w_packed.device)
    fn = lib.segquant_unpack_weight if bits == 8 else lib.segquant_unpack_weight_w4
    _check(fn(_ptr(w_packed), K, N, _ptr(out), _ld(out, "out"), _stream(w_packed)),
           "segquant_unpack_weight" + ("" if bits == 8 else "_w4"))
    return out


def segquant_gemm_workspace_bytes(M: int, N: int, K: int, kseg: Optional[Sequence[int]] = None,
                                  flags: int = SEGQ_GEMM_AUTO) -> int:
    off, wid = _segs(kseg, K)
    return int(load_library().segquant_gemm_workspace_bytes(M, N, K, len(wid), _arr_ptr(off),
                                                            _arr_ptr(wid), flags))


def segquant_gemm_w8a8_seg(x, w_packed, w_scale, act_scales, kseg: Optional[Sequence[int]] = None,
                           N: Optional[int] = None, xq=None, q_layout: int = SEGQ_Q_SIGNED,
                           out=None, acc_debug=None, workspace="auto",
                           flags: int = SEGQ_GEMM_AUTO):
    """The DualScale x SegLinear W8A8 layer (one launch, or quantisation
    then GEMM when a workspace is given and the library asks for one).

    x: bf16 [M][K] (or None with xq = the output of
    segquant_quantize_dualscale); w_packed/w_scale from
    segquant_quantize_weight; act_scales from segquant_calibrate_amax.
    Returns bf16 Y [M][N].  acc_debug, if given, is an int32 tensor
    [2][n_kseg][M][N] that receives the per-segment accumulators.
    workspace: a device tensor, None (always the fused launch), or "auto"
    (a tensor of segquant_gemm_workspace_bytes() bytes from torch's
    allocator when that is nonzero)."""
    import torch
    lib = load_library()
    src = x if x is not None else xq
    if x is not None:
        M, K = x.shape
        ld_x, ld_q = _ld(x, "x"), 0
    else:
        M = xq.shape[-2]
        K = sum(kseg) if kseg is not None else None
        if K is None:
            raise ValueError("kseg is required with a pre-quantised input")
        ld_x, ld_q = 0, xq.stride(-2)
    if N is None:
        N = w_scale.shape[1]
    off, wid = _segs(kseg, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=src.device)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be a tensor, None or 'auto'")
        nb = segquant_gemm_workspace_bytes(M, N, K, kseg, flags)
        workspace = torch.empty(nb, dtype=torch.uint8, device=src.device) if nb else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.segquant_gemm_w8a8_seg(M, N, K, _ptr(x), ld_x, _ptr(xq), ld_q, q_layout,
                                      _ptr(w_packed), _ptr(w_scale), len(wid), _arr_ptr(off),
                                      _arr_ptr(wid), _ptr(act_scales), _ptr(out), _ld(out, "out"),
                                      _ptr(acc_debug), _ptr(workspace), ws_bytes, flags,
                                      _stream(src)),
           "segquant_gemm_w8a8_seg")
    return out


def segquant_gemm_w8a8_seg_noalloc(x, w_packed, w_scale, act_scales, out,
                                   kseg: Optional[Sequence[int]] = None, N: Optional[int] = None,
                                   xq=None, q_layout: int = SEGQ_Q_SIGNED, acc_debug=None,
                                   flags: int = SEGQ_GEMM_AUTO):
    """segquant_gemm_w8a8_seg through its no-allocation entry point: no
    workspace, no device allocation in the call (the library's own scratch
    array stands in for the workspace).  `out` (bf16 [M][N]) is required:
    this path allocates nothing, here or in the library."""
    lib = load_library()
    src = x if x is not None else xq
    if x is not None:
        M, K = x.shape
        ld_x, ld_q = _ld(x, "x"), 0
    else:
        M = xq.shape[-2]
        if kseg is None:
            raise ValueError("kseg is required with a pre-quantised input")
        K = sum(kseg)
        ld_x, ld_q = 0, xq.stride(-2)
    if N is None:
        N = w_scale.shape[1]
    off, wid = _segs(kseg, K)
    _check(lib.segquant_gemm_w8a8_seg_noalloc(M, N, K, _ptr(x), ld_x, _ptr(xq), ld_q, q_layout,
                                              _ptr(w_packed), _ptr(w_scale), len(wid),
                                              _arr_ptr(off), _arr_ptr(wid), _ptr(act_scales),
                                              _ptr(out), _ld(out, "out"), _ptr(acc_debug), flags,
                                              _stream(src)),
           "segquant_gemm_w8a8_seg_noalloc")
    return out
