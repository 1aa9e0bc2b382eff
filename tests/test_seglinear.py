"""SegLinear segment discovery on small synthetic modules (CPU).

[P1] "SegLinear" section; [P2] section 2 and the graph-to-kernel workflow:
linear -> chunk/split gives N-segments, concat or a head-merging reshape ->
linear gives K-segments, widths from the graph's shape metadata.  The toy
modules mirror the layers the benchmark workloads stand for (a DiT AdaNorm
projection chunked into six modulation vectors, an attention output
projection after merging heads), so the discovered lists are checked
against those workloads' segment lists too.
"""
import pytest
import torch
import torch.nn as nn
import torch.nn.functional as F

from segmented_dual_scale_amd import seglinear
from segmented_dual_scale_amd import workloads as W


class AdaNorm(nn.Module):
    """Timestep embedding -> SiLU -> linear -> six modulation vectors
    (shift, scale, gate for two branches)."""

    def __init__(self, d):
        super().__init__()
        self.lin = nn.Linear(d, 6 * d)

    def forward(self, emb):
        return self.lin(F.silu(emb)).chunk(6, dim=1)


class AttnOut(nn.Module):
    """(B, H, T, D) heads -> (B, T, H*D) -> output projection."""

    def __init__(self, heads, dh, d):
        super().__init__()
        self.h, self.dh = heads, dh
        self.proj = nn.Linear(heads * dh, d)

    def forward(self, o):
        b, h, t, dh = o.shape
        return self.proj(o.transpose(1, 2).reshape(b, t, h * dh))


class Skip(nn.Module):
    """Concat of a skip connection and the main path, then a linear whose
    output is split unevenly."""

    def __init__(self):
        super().__init__()
        self.fuse = nn.Linear(128 + 384, 256)

    def forward(self, a, b):
        y = self.fuse(torch.cat([a, b], dim=-1))
        p, q = torch.split(y, [64, 192], dim=-1)
        return p, q


class Plain(nn.Module):
    def __init__(self):
        super().__init__()
        self.fc1 = nn.Linear(64, 256)
        self.fc2 = nn.Linear(256, 64)

    def forward(self, x):
        h = self.fc1(x)
        a, b = h.chunk(2, dim=0)          # along the batch: not a feature boundary
        return self.fc2(F.gelu(torch.cat([a, b], dim=0)))


class Nested(nn.Module):
    def __init__(self):
        super().__init__()
        self.block = nn.Sequential(nn.Linear(64, 192))
        self.out = nn.Linear(64, 64)

    def forward(self, x):
        q, k, v = self.block(x).split(64, dim=-1)
        return self.out(q * k + v)


def test_output_segmented_chunk_matches_the_adanorm_workload():
    wl = W.WORKLOADS["c2_adanorm_gemv"]
    d = wl.K
    plans = seglinear.discover(AdaNorm(d), torch.randn(wl.M, d))
    p = plans["lin"]
    assert p.nseg == list(wl.nseg) == [d] * 6 and p.kseg is None
    assert p.patterns == ["linear->chunk/split"] and p.kernel_ready()


def test_input_segmented_head_merge_matches_the_attention_workload():
    wl = W.WORKLOADS["c4_attn_out_inseg"]
    heads, dh = len(wl.kseg), wl.kseg[0]
    plans = seglinear.discover(AttnOut(heads, dh, wl.N), torch.randn(1, heads, 7, dh))
    p = plans["proj"]
    assert p.kseg == list(wl.kseg) == [64] * 24 and p.nseg is None
    assert p.kernel_ready()


def test_concat_then_uneven_split():
    plans = seglinear.discover(Skip(), torch.randn(3, 5, 128), torch.randn(3, 5, 384))
    p = plans["fuse"]
    assert p.kseg == [128, 384] and p.nseg == [64, 192]
    assert set(p.patterns) == {"concat->linear", "linear->chunk/split"}
    assert p.kernel_ready()


def test_no_feature_boundary_means_no_segments():
    plans = seglinear.discover(Plain(), torch.randn(4, 64))
    assert plans["fc1"].nseg is None and plans["fc1"].kseg is None
    assert plans["fc2"].kseg is None and plans["fc2"].nseg is None


def test_nested_names_and_int_split():
    plans = seglinear.discover(Nested(), torch.randn(2, 64))
    assert plans["block.0"].nseg == [64, 64, 64]
    assert plans["out"].kseg is None


@pytest.mark.parametrize("n,chunks,want", [(10, 3, [4, 4, 2]), (9, 4, [3, 3, 3]), (12, 5, [3, 3, 3, 3])])
def test_chunk_widths_follow_torch(n, chunks, want):
    assert seglinear._chunk_widths(n, chunks) == want
    assert [t.shape[0] for t in torch.arange(n).chunk(chunks)] == want


@pytest.mark.parametrize("n,spec", [(10, 4), (9, 4), (12, 3), (10, [3, 7])])
def test_split_widths_follow_torch(n, spec):
    assert seglinear._split_widths(n, spec) == [t.shape[0] for t in torch.arange(n).split(spec)]


def test_kernel_ready_rejects_misaligned_k_boundaries():
    assert not seglinear.SegPlan(in_features=512, out_features=256, kseg=[100, 412]).kernel_ready()
    assert seglinear.SegPlan(in_features=512, out_features=256, kseg=[128, 384]).kernel_ready()
    assert not seglinear.SegPlan(in_features=512, out_features=250).kernel_ready()


def test_linear_called_twice_gets_two_plans():
    class Twice(nn.Module):
        def __init__(self):
            super().__init__()
            self.l = nn.Linear(64, 128)

        def forward(self, x, y):
            return self.l(x).chunk(2, dim=-1)[0], self.l(torch.cat([y, y], dim=-1))

    plans = seglinear.discover(Twice(), torch.randn(2, 64), torch.randn(2, 32))
    assert plans["l#1"].nseg == [64, 64] and plans["l#1"].kseg is None
    assert plans["l#2"].kseg == [32, 32] and plans["l#2"].nseg is None
