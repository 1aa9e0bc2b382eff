"""Kernel dispatches per layer call, counted in a captured HIP graph.

The pages run both polarity products as one batched launch with the scale
combine in its epilogue ([P1] "DualScale", hardware-native execution; [P2]
section 3).  Here a call is captured (not run) and the kernel nodes of the
graph are counted through the HIP runtime that torch and the library share:
the fused call is exactly one kernel, for every workload shape; with a
workspace the library may first quantise into it (then exactly two).  No
call records a memset node."""
import ctypes

import pytest

import segmented_dual_scale_amd as S
from segmented_dual_scale_amd import workloads as W

pytestmark = pytest.mark.gpu

HIP_GRAPH_NODE_KERNEL = 0
HIP_GRAPH_NODE_MEMSET = 2


def _hip():
    path = None
    with open("/proc/self/maps") as fh:
        for ln in fh:
            if "libamdhip64.so" in ln:
                path = ln.split()[-1]
                break
    assert path, "the HIP runtime is not loaded"
    lib = ctypes.CDLL(path)  # the already-loaded runtime (same handle)
    lib.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    return lib


def node_types(fn):
    import torch
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(g, stream=stream):
        fn()
    h = ctypes.c_void_p(g.raw_cuda_graph())
    hip = _hip()
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(h, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * max(1, n.value))()
    assert hip.hipGraphGetNodes(h, nodes, ctypes.byref(n)) == 0
    kinds = []
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
        kinds.append(t.value)
    del g
    return kinds


@pytest.mark.parametrize("name", W.ORDER)
@pytest.mark.parametrize("mode", ["fused", "auto"])
def test_dispatches_per_call(name, mode):
    import torch
    wl = W.WORKLOADS[name]
    dev = "cuda:0"
    # shapes only: a captured call is recorded, not run
    x = torch.zeros((wl.M, wl.K), dtype=torch.bfloat16, device=dev)
    wp = torch.zeros(S.segquant_weight_packed_bytes(wl.K, wl.N), dtype=torch.int8, device=dev)
    ws = torch.zeros((len(wl.kseg), wl.N), dtype=torch.float32, device=dev)
    act = torch.zeros((4, len(wl.kseg)), dtype=torch.float32, device=dev)
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
    flags = S.SEGQ_GEMM_FUSED_QUANT if mode == "fused" else S.SEGQ_GEMM_AUTO
    nb = S.segquant_gemm_workspace_bytes(wl.M, wl.N, wl.K, list(wl.kseg), flags)
    work = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def call():
        S.segquant_gemm_w8a8_seg(x, wp, ws, act, list(wl.kseg), out=y,
                                 workspace=work if nb else None, flags=flags)

    kinds = node_types(call)
    assert HIP_GRAPH_NODE_MEMSET not in kinds
    expect = 1 if nb == 0 else 2
    if mode == "fused":
        assert nb == 0
    assert kinds.count(HIP_GRAPH_NODE_KERNEL) == expect, (name, mode, kinds)
