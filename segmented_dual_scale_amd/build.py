"""Build libsegquant.so (gfx950) in-tree with hipcc.

    python -m segmented_dual_scale_amd.build

Every source compiles with -ffp-contract=off (the quantisation multiplies
and rounding adds must stay separate IEEE operations) and with packed fp32
VALU instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OUT = os.path.join(HERE, "libsegquant.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "act_kernels.hip", "weight_kernels.hip", "gemm_tile.hip", "gemm_lds.hip",
           "gemm_smallm.hip", "noalloc.hip"]
# ceiling probes for the benchmark (matrix-core-only loop, streaming read):
# a library of their own, not part of the layer's
PROBE_SOURCES = ["probes.hip"]
PROBE_OUT = os.path.join(HERE, "libsegquant_probe.so")

ARCH = os.environ.get("SEGQUANT_ARCH", "gfx950")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-I", INCLUDE,
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def object_path(src: str) -> str:
    return os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")


def compile_source(src: str, out: str | None = None, extra_flags=None, verbose: bool = False) -> str:
    """Compile one source of csrc/ to an object file (default: _build/<name>.o)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = out or object_path(src)
    cmd = [_hipcc(), *CFLAGS, *(extra_flags or []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def link_shared(out: str, objs, extra_flags=None) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *(extra_flags or []), "-o", tmp,
           *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: compile_source(f, extra_flags=extra_flags, verbose=verbose),
                           srcs))
    link_shared(OUT, objs[:len(SOURCES)])
    link_shared(PROBE_OUT, objs[len(SOURCES):])
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
