"""SegLinear segment discovery: the K- and N-segment lists of every linear
layer of a module, read off its static graph.

[P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
     for Diffusion Models" (papernotes.org notes), "SegLinear" section: the
     torch.fx graph is searched for chunk/split after a linear (output-
     segmented) and concat/reshape before one (input-segmented).
[P2] "SegQuant" (hliangzhao.me), section 2 and the graph-to-kernel workflow:
     trace the graph with shapes, match concat-to-linear and linear-to-split,
     take the segment widths from the graph metadata.

This is host-side planning, the step before the layer: it produces the
`kseg` / `nseg` lists that segquant_quantize_weight and
segquant_gemm_w8a8_seg take.  Nothing here runs on the GPU or reads data
beyond the example inputs' shapes.

Patterns (the last dimension is the feature dimension of a linear):
  output-segmented  linear -> chunk(c, dim=-1) or split(sizes, dim=-1)
                    -> N-segments: the chunk/split widths
  input-segmented   cat([a, b, ...], dim=-1) -> linear
                    -> K-segments: the last-dimension widths of the parts
                    reshape/view/flatten merging (..., H, D) into (..., H*D)
                    -> linear (the multi-head merge before an attention's
                    output projection)
                    -> K-segments: H segments of width D
A linear used by several consumers is output-segmented only if one of them
is such a chunk/split.  Reading of a point the pages leave open: a chunk or
split along another dimension, or a reshape that does not merge the last two
dimensions, is not a semantic boundary of the feature dimension and is
ignored.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch
import torch.fx
from torch.fx.passes.shape_prop import ShapeProp


@dataclass
class SegPlan:
    """Segments of one linear layer (None: a single segment)."""
    in_features: int
    out_features: int
    kseg: Optional[List[int]] = None   # K-segment widths, input-segmented
    nseg: Optional[List[int]] = None   # N-segment widths, output-segmented
    patterns: List[str] = field(default_factory=list)

    def kernel_ready(self) -> bool:
        """Whether the lists fit the GEMM's layout rules: K-segment
        boundaries on multiples of 64, N a multiple of 16."""
        if self.out_features % 16 or self.in_features % 64:
            return False
        if self.kseg:
            edges = 0
            for w in self.kseg[:-1]:
                edges += w
                if edges % 64:
                    return False
        return True


def _shape(node) -> Optional[torch.Size]:
    meta = node.meta.get("tensor_meta")
    return getattr(meta, "shape", None)


def _last_dim(dim, ndim: int) -> bool:
    return dim == -1 or dim == ndim - 1


def _arg(node, pos: int, name: str, default=None):
    if len(node.args) > pos:
        return node.args[pos]
    return node.kwargs.get(name, default)


def _chunk_widths(n: int, chunks: int) -> List[int]:
    # torch.chunk: pieces of ceil(n / chunks), the last one smaller (and
    # possibly fewer pieces than asked for)
    size = -(-n // chunks)
    out, left = [], n
    while left > 0:
        out.append(min(size, left))
        left -= size
    return out


def _split_widths(n: int, spec) -> List[int]:
    # torch.split: an int gives pieces of that size (the last one smaller),
    # a list gives the sizes themselves
    if isinstance(spec, int):
        if spec <= 0:
            return [n]
        return [spec] * (n // spec) + ([n % spec] if n % spec else [])
    return [int(w) for w in spec]


def _is(node, op: str, *targets) -> bool:
    if node.op != op:
        return False
    return node.target in targets


def _output_segments(lin_node, n: int) -> Optional[List[int]]:
    ndim = len(_shape(lin_node))
    for user in lin_node.users:
        if _is(user, "call_method", "chunk") or _is(user, "call_function", torch.chunk):
            chunks = _arg(user, 1, "chunks")
            if isinstance(chunks, int) and _last_dim(_arg(user, 2, "dim", 0), ndim):
                widths = _chunk_widths(n, chunks)
                if len(widths) > 1:
                    return widths
        if _is(user, "call_method", "split") or _is(user, "call_function", torch.split):
            spec = _arg(user, 1, "split_size_or_sections", _arg(user, 1, "split_size"))
            if spec is not None and _last_dim(_arg(user, 2, "dim", 0), ndim):
                widths = _split_widths(n, spec)
                if len(widths) > 1:
                    return widths
    return None


_CATS = (torch.cat, torch.concat)
_RESHAPES = ("reshape", "view", "flatten")


def _input_segments(src, k: int):
    """(widths, pattern) for the node feeding a linear, or (None, None)."""
    if _is(src, "call_function", *_CATS):
        parts = _arg(src, 0, "tensors")
        out_shape = _shape(src)
        if out_shape is not None and isinstance(parts, (list, tuple)) and \
                _last_dim(_arg(src, 1, "dim", 0), len(out_shape)):
            widths = [int(_shape(p)[-1]) for p in parts]
            if len(widths) > 1 and sum(widths) == k:
                return widths, "concat->linear"
    is_reshape = (src.op == "call_method" and src.target in _RESHAPES) or \
        _is(src, "call_function", torch.reshape, torch.flatten)
    if is_reshape and src.args:
        inp = src.args[0]
        in_shape, out_shape = _shape(inp), _shape(src)
        if in_shape is not None and out_shape is not None and len(in_shape) >= 2 and \
                int(out_shape[-1]) == k and int(in_shape[-2]) * int(in_shape[-1]) == k and \
                int(in_shape[-1]) != k:
            heads, width = int(in_shape[-2]), int(in_shape[-1])
            return [width] * heads, "reshape(H, D -> H*D)->linear"
    return None, None


def discover(module: torch.nn.Module, *example_inputs) -> Dict[str, SegPlan]:
    """Trace `module` symbolically, propagate the example inputs' shapes and
    return a SegPlan for every nn.Linear call (keyed by its qualified
    module name; a linear called twice gets '#1', '#2' ... suffixes).
    Functional linears (F.linear) are not linear layers with weights of
    their own here and are not reported."""
    gm = torch.fx.symbolic_trace(module)
    ShapeProp(gm).propagate(*example_inputs)
    mods = dict(gm.named_modules())
    plans: Dict[str, SegPlan] = {}
    seen: Dict[str, int] = {}
    for node in gm.graph.nodes:
        if node.op != "call_module" or not isinstance(mods.get(node.target), torch.nn.Linear):
            continue
        lin = mods[node.target]
        plan = SegPlan(in_features=lin.in_features, out_features=lin.out_features)
        widths = _output_segments(node, lin.out_features)
        if widths:
            plan.nseg = widths
            plan.patterns.append("linear->chunk/split")
        kw, pat = _input_segments(node.args[0], lin.in_features)
        if kw:
            plan.kseg = kw
            plan.patterns.append(pat)
        name = node.target
        seen[name] = seen.get(name, 0) + 1
        if seen[name] > 1:
            if seen[name] == 2:
                plans[name + "#1"] = plans.pop(name)
            name = f"{name}#{seen[name]}"
        plans[name] = plan
    return plans
