"""CPU oracle for the DualScale x SegLinear W8A8 linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``segmented_dual_scale_amd``) never imports, loads or calls it, and
the two share no code: the only thing both sides use is the seeded input
generator module ``segmented_dual_scale_amd.workloads``, which holds none of
the method's arithmetic.

The arithmetic lives in ``segquant_oracle.c`` (plain C, OpenMP over output
rows); this module compiles it with gcc and wraps it for numpy arrays.  The
citations of the pages sit beside each C function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "segquant_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# SEGQUANT_ORACLE_LIBRARY names another build of the same source (the
# sanitizer test builds one with address and undefined-behaviour checks).
_LIB_OVERRIDE = os.environ.get("SEGQUANT_ORACLE_LIBRARY")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` next to its source (gcc, -O2, no fast-math,
    no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_polarity_split.restype = None
    lib.oracle_polarity_split.argtypes = [P, I64, P, P]
    lib.oracle_calibrate_amax.argtypes = [P, I64, I64, I64, I32, P, P, P, P, P, P]
    lib.oracle_calibrate_amax_single.argtypes = [P, I64, I64, I64, I32, P, P, P, P, P, P]
    lib.oracle_activation.argtypes = [P, I64, I32, P]
    lib.oracle_quantize_dualscale.argtypes = [P, I64, I64, I64, I32, P, P, P, P, P, P]
    lib.oracle_quantize_weight.argtypes = [P, I64, I64, I64, I32, P, P, I32, P, P, I32, P, P]
    lib.oracle_quantize_weight_w4.argtypes = [P, I64, I64, I64, I32, P, P, I32, P, P, I32, P, P]
    lib.oracle_segment_acc.argtypes = [P, P, P, I64, I64, I64, I32, P, P, P]
    lib.oracle_dequantize.argtypes = [P, I64, I64, I32, P, P, P, P]
    lib.oracle_dualscale_linear.argtypes = [P, I64, I64, I64, P, P, I64, I32, P, P, P, P, P, P, P]
    for f in ("oracle_calibrate_amax", "oracle_calibrate_amax_single", "oracle_activation",
              "oracle_quantize_dualscale", "oracle_quantize_weight", "oracle_quantize_weight_w4",
              "oracle_segment_acc", "oracle_dequantize", "oracle_dualscale_linear"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _segs(widths: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    w = np.ascontiguousarray(np.asarray(widths, dtype=np.int32))
    off = np.zeros_like(w)
    if len(w) > 1:
        off[1:] = np.cumsum(w)[:-1]
    return off, w


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def polarity_split(x_bf16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    xp = np.empty(x.shape, np.float32)
    xn = np.empty(x.shape, np.float32)
    _load().oracle_polarity_split(_ptr(x), x.size, _ptr(xp), _ptr(xn))
    return xp, xn


def calibrate_amax(x_bf16: np.ndarray, kseg: Sequence[int]):
    """Returns (s_pos, s_neg, inv_pos, inv_neg), each fp32 [n_kseg]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    off, wid = _segs(kseg)
    out = [np.empty(len(wid), np.float32) for _ in range(4)]
    _check(_load().oracle_calibrate_amax(_ptr(x), M, K, K, len(wid), _ptr(off), _ptr(wid),
                                         *[_ptr(o) for o in out]), "calibrate_amax")
    return tuple(out)


def activation(z_bf16: np.ndarray, kind: str) -> np.ndarray:
    """SiLU ("silu") or exact GELU ("gelu") of bf16 values, in fp64."""
    z = np.ascontiguousarray(z_bf16, dtype=np.uint16)
    out = np.empty(z.shape, np.float64)
    _check(_load().oracle_activation(_ptr(z), z.size, {"silu": 1, "gelu": 2}[kind], _ptr(out)),
           "activation")
    return out


def calibrate_amax_single(x_bf16: np.ndarray, kseg: Sequence[int]):
    """Single-scale table: (s, s, inv, inv) per K-segment, s = max|x|/127."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    off, wid = _segs(kseg)
    out = [np.empty(len(wid), np.float32) for _ in range(4)]
    _check(_load().oracle_calibrate_amax_single(_ptr(x), M, K, K, len(wid), _ptr(off), _ptr(wid),
                                                *[_ptr(o) for o in out]), "calibrate_amax_single")
    return tuple(out)


def quantize_dualscale(x_bf16: np.ndarray, kseg: Sequence[int], inv_pos, inv_neg):
    """Returns the two int8 planes (q_pos, q_neg), each [M][K]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, K = x.shape
    off, wid = _segs(kseg)
    ip = np.ascontiguousarray(inv_pos, dtype=np.float32)
    ineg = np.ascontiguousarray(inv_neg, dtype=np.float32)
    qp = np.empty((M, K), np.int8)
    qn = np.empty((M, K), np.int8)
    _check(_load().oracle_quantize_dualscale(_ptr(x), M, K, K, len(wid), _ptr(off), _ptr(wid),
                                             _ptr(ip), _ptr(ineg), _ptr(qp), _ptr(qn)),
           "quantize_dualscale")
    return qp, qn


def quantize_weight(w: np.ndarray, kseg: Sequence[int], nseg: Sequence[int] | None,
                    per_column: bool, bits: int = 8):
    """Returns (w_q int8 [K][N], w_scale fp32 [n_kseg][N]); bits=4: the
    4-bit weights (codes in [-7, 7], s_w = amax/7)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    koff, kwid = _segs(kseg)
    if nseg is None:
        nseg = [N]
    noff, nwid = _segs(nseg)
    wq = np.empty((K, N), np.int8)
    ws = np.empty((len(kwid), N), np.float32)
    fn = {8: _load().oracle_quantize_weight, 4: _load().oracle_quantize_weight_w4}[bits]
    _check(fn(_ptr(w), K, N, N, len(kwid), _ptr(koff), _ptr(kwid), len(nwid), _ptr(noff),
              _ptr(nwid), int(per_column), _ptr(wq), _ptr(ws)), "quantize_weight")
    return wq, ws


def segment_acc(q_pos: np.ndarray, q_neg: np.ndarray, w_q: np.ndarray, kseg: Sequence[int]):
    """Returns int32 acc[2][n_kseg][M][N] (half 0 = +, half 1 = -)."""
    qp = np.ascontiguousarray(q_pos, dtype=np.int8)
    qn = np.ascontiguousarray(q_neg, dtype=np.int8)
    wq = np.ascontiguousarray(w_q, dtype=np.int8)
    M, K = qp.shape
    K2, N = wq.shape
    assert K == K2 and qn.shape == qp.shape
    off, wid = _segs(kseg)
    acc = np.empty((2, len(wid), M, N), np.int32)
    _check(_load().oracle_segment_acc(_ptr(qp), _ptr(qn), _ptr(wq), M, K, N, len(wid),
                                      _ptr(off), _ptr(wid), _ptr(acc)), "segment_acc")
    return acc


def dequantize(acc: np.ndarray, s_pos, s_neg, w_scale: np.ndarray) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    _, S, M, N = acc.shape
    sp = np.ascontiguousarray(s_pos, dtype=np.float32)
    sn = np.ascontiguousarray(s_neg, dtype=np.float32)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    assert ws.shape == (S, N) and sp.shape == (S,) and sn.shape == (S,)
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_dequantize(_ptr(acc), M, N, S, _ptr(sp), _ptr(sn), _ptr(ws), _ptr(y)),
           "dequantize")
    return y


def dualscale_linear(x_bf16: np.ndarray, w_q: np.ndarray, w_scale: np.ndarray,
                     kseg: Sequence[int], s_pos, s_neg, inv_pos, inv_neg) -> np.ndarray:
    """The whole layer (quantise -> per-segment int32 products -> fp64
    dequantisation), row by row.  Returns fp64 Y [M][N]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    wq = np.ascontiguousarray(w_q, dtype=np.int8)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = x.shape
    _, N = wq.shape
    off, wid = _segs(kseg)
    arrs = [np.ascontiguousarray(a, dtype=np.float32) for a in (s_pos, s_neg, inv_pos, inv_neg)]
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_dualscale_linear(_ptr(x), M, K, K, _ptr(wq), _ptr(ws), N, len(wid),
                                           _ptr(off), _ptr(wid), *[_ptr(a) for a in arrs],
                                           _ptr(y)), "dualscale_linear")
    return y
