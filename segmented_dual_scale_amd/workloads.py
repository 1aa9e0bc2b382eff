"""Seeded synthetic workloads for the DualScale x SegLinear W8A8 layer.

This module only draws inputs: activations X (returned as bf16 bit patterns,
uint16 [M][K]) and fp32 weights W [K][N], plus each workload's segment lists.
It holds none of the method's arithmetic (no calibration, quantisation,
products or rescaling), so both the HIP path and the CPU oracle may use it.

The five named workloads take the layer shapes the pages quantise and the
polarity structure of their activation statistics:
  * [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization
    Framework for Diffusion Models" (papernotes.org notes): the
    activation-polarity table in the "DualScale" section (AdaNorm/SiLU with
    about 95 % negative-dominant channels, FFN/GELU), the stated value ranges
    (positive up to about 3.5, negative within [-0.3, 0]), the AdaNorm
    shift/scale chunking (output-segmented) and the multi-head concat
    (input-segmented) of the SegLinear section.
  * [P2] "SegQuant" (hliangzhao.me): section 1, AdaNorm emits shift, scale and
    gate for the attention and MLP branches (six output segments).
No dataset item is used: every number comes from a seeded generator.

Generator: numpy PCG64 seeded by SeedSequence([seed, workload index,
tensor id]); tensor ids are 0 per-channel parameters, 1 activation noise,
2 per-segment weight spreads, 3 weight noise.  SiLU/GELU (exact erf form)
are applied in fp32 and the result is rounded once to bf16 (ties to even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    M: int
    K: int
    N: int
    kseg: Tuple[int, ...]          # K-segment widths (input-segmented); (K,) if none
    nseg: Tuple[int, ...]          # N-segment widths for weight-scale groups
    per_column: bool               # one weight scale per output column (per K-segment)
    description: str = field(default="", compare=False)


WORKLOADS = {
    "c1_tiny_outseg": Workload(
        "c1_tiny_outseg", 1, 64, 256, 768, (256,), (256, 256, 256), False,
        "Tiny output-segmented layer: X = SiLU(z), z ~ N(0,1); W columns in 3 segments of 256 "
        "with sigma (0.02, 0.1, 0.5); one weight scale per segment; one global s+/s-"),
    "c2_adanorm_gemv": Workload(
        "c2_adanorm_gemv", 2, 2, 1536, 9216, (1536,), (1536,) * 6, False,
        "AdaNorm-shaped small-M layer: X = SiLU(t), t_j ~ N(mu_j, 1), mu = -1.5 on 95% of "
        "channels and +1.0 on the rest; W in 6 column segments (shift/scale/gate x2) with "
        "log-uniform sigma in [0.01, 0.3]"),
    "c3_dit_ffn_fc2": Workload(
        "c3_dit_ffn_fc2", 3, 4096, 6144, 1536, (6144,), (1536,), True,
        "DiT FFN fc2, no segments: X = GELU(z), z_mj ~ N(0, sigma_j), sigma_j log-normal(0, 0.5), "
        "1% outlier channels x8; W ~ N(0, 0.02); per-output-column weight scale"),
    "c4_attn_out_inseg": Workload(
        "c4_attn_out_inseg", 4, 4429, 1536, 1536, (64,) * 24, (1536,), False,
        "Input-segmented attention out-projection: 4096 image + 333 text tokens; X = 24 head "
        "blocks of width 64, block h ~ N(0, sigma_h), sigma_h log-uniform in [0.2, 4]; one "
        "weight scale and one s+/s- pair per K-segment"),
    "c5_flux_ffn_fc2": Workload(
        "c5_flux_ffn_fc2", 5, 9216, 12288, 3072, (3072,) * 4, (3072,), False,
        "FLUX-width FFN fc2 (2 x 4608 tokens): X = GELU(z), z_mj ~ N(0, sigma_j), sigma_j "
        "log-normal(0, 0.5); W ~ N(0, 0.02) in 4 row segments with their own scales"),
}

ORDER: List[str] = list(WORKLOADS)


def rng_for(seed: int, index: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index, tensor_id])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, ties to even (finite inputs), returning the bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _silu(a: np.ndarray) -> np.ndarray:
    import torch
    return torch.nn.functional.silu(torch.from_numpy(a)).numpy()


def _gelu(a: np.ndarray) -> np.ndarray:
    import torch
    return torch.nn.functional.gelu(torch.from_numpy(a)).numpy()


def _normal(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float32)


def make_x(wl: Workload, seed: int = 0) -> np.ndarray:
    """Activation X of a named workload as bf16 bits, uint16 [M][K]."""
    M, K = wl.M, wl.K
    g0, g1 = rng_for(seed, wl.index, 0), rng_for(seed, wl.index, 1)
    if wl.index == 1:
        x = _silu(_normal(g1, (M, K)))
    elif wl.index == 2:
        n_neg = int(math.floor(0.95 * K))
        mu = np.full(K, 1.0, np.float32)
        mu[g0.permutation(K)[:n_neg]] = -1.5
        x = _silu(_normal(g1, (M, K)) + mu[None, :])
    elif wl.index in (3, 5):
        sigma = g0.lognormal(0.0, 0.5, K).astype(np.float32)
        if wl.index == 3:
            sigma[g0.permutation(K)[: int(math.floor(0.01 * K))]] *= 8.0
        z = _normal(g1, (M, K))
        z *= sigma[None, :]
        x = _gelu(z)
    elif wl.index == 4:
        nh = len(wl.kseg)
        sig_h = np.exp(g0.uniform(math.log(0.2), math.log(4.0), nh)).astype(np.float32)
        x = _normal(g1, (M, K))
        x *= np.repeat(sig_h, K // nh)[None, :]
    else:
        raise ValueError(wl.name)
    return f32_to_bf16_bits(x)


def preact_kind(wl: Workload) -> Optional[str]:
    """Activation that produces the workload's X from its pre-activation:
    "silu" (c1, c2), "gelu" (c3, c5), or None (c4 has no activation)."""
    return {1: "silu", 2: "silu", 3: "gelu", 5: "gelu"}.get(wl.index)


def make_preact(wl: Workload, seed: int = 0) -> np.ndarray:
    """The pre-activation z of an activation workload as bf16 bits [M][K]:
    the same draws make_x passes through SiLU/GELU, rounded to bf16 (the
    input of the producer-fused quantisation; X there is bf16(act(bf16 z)))."""
    M, K = wl.M, wl.K
    g0, g1 = rng_for(seed, wl.index, 0), rng_for(seed, wl.index, 1)
    if wl.index == 1:
        z = _normal(g1, (M, K))
    elif wl.index == 2:
        n_neg = int(math.floor(0.95 * K))
        mu = np.full(K, 1.0, np.float32)
        mu[g0.permutation(K)[:n_neg]] = -1.5
        z = _normal(g1, (M, K)) + mu[None, :]
    elif wl.index in (3, 5):
        sigma = g0.lognormal(0.0, 0.5, K).astype(np.float32)
        if wl.index == 3:
            sigma[g0.permutation(K)[: int(math.floor(0.01 * K))]] *= 8.0
        z = _normal(g1, (M, K))
        z *= sigma[None, :]
    else:
        raise ValueError(f"{wl.name} has no activation")
    return f32_to_bf16_bits(z)


def make_w(wl: Workload, seed: int = 0) -> np.ndarray:
    """Weight W of a named workload, fp32 [K][N]."""
    K, N = wl.K, wl.N
    g2, g3 = rng_for(seed, wl.index, 2), rng_for(seed, wl.index, 3)
    w = _normal(g3, (K, N))
    if wl.index == 1:
        col_sigma = np.repeat(np.array([0.02, 0.1, 0.5], np.float32), 256)
    elif wl.index == 2:
        seg_sigma = np.exp(g2.uniform(math.log(0.01), math.log(0.3), len(wl.nseg)))
        col_sigma = np.repeat(seg_sigma.astype(np.float32), wl.nseg[0])
    else:
        col_sigma = np.full(N, 0.02, np.float32)
    w *= col_sigma[None, :]
    return w


def make_inputs(name: str, seed: int = 0) -> Tuple[Workload, np.ndarray, np.ndarray]:
    wl = WORKLOADS[name]
    return wl, make_x(wl, seed), make_w(wl, seed)


def make_custom(M: int, K: int, N: int, seed: int, kind: str = "gelu",
                x_scale: float = 1.0, w_sigma: float = 0.05) -> Tuple[np.ndarray, np.ndarray]:
    """Free-shape inputs for edge cases and small parity runs.

    kind: "gelu" (GELU of N(0, x_scale^2), skewed negative tail), "silu",
    "normal" (symmetric), "pos" (all >= 0), "neg" (all <= 0),
    "blocks" (per-64-column spreads as in the attention workload)."""
    g0, g1, g3 = rng_for(seed, 100, 0), rng_for(seed, 100, 1), rng_for(seed, 100, 3)
    z = _normal(g1, (M, K)) * np.float32(x_scale)
    if kind == "gelu":
        x = _gelu(z)
    elif kind == "silu":
        x = _silu(z)
    elif kind == "normal":
        x = z
    elif kind == "pos":
        x = np.abs(z)
    elif kind == "neg":
        x = -np.abs(z)
    elif kind == "blocks":
        nb = max(1, (K + 63) // 64)
        sig = np.exp(g0.uniform(math.log(0.2), math.log(4.0), nb)).astype(np.float32)
        x = z * np.repeat(sig, 64)[None, :K]
    else:
        raise ValueError(kind)
    w = _normal(g3, (K, N)) * np.float32(w_sigma)
    return f32_to_bf16_bits(x), w


def even_segments(total: int, n: int, align: int = 64) -> Tuple[int, ...]:
    """n widths that cover `total`, every boundary a multiple of `align`."""
    blocks = total // align
    assert blocks * align == total and 1 <= n <= blocks
    base, extra = divmod(blocks, n)
    return tuple((base + (1 if i < extra else 0)) * align for i in range(n))


def random_segments(total: int, rng: np.random.Generator, max_n: Optional[int] = None,
                    align: int = 64) -> Tuple[int, ...]:
    """A random segment list covering `total` with boundaries on `align`."""
    blocks = total // align
    assert blocks * align == total and blocks >= 1
    n = int(rng.integers(1, min(blocks, max_n or blocks) + 1))
    cuts = np.sort(rng.choice(np.arange(1, blocks), size=n - 1, replace=False)) if n > 1 else []
    edges = [0, *[int(c) for c in cuts], blocks]
    return tuple((edges[i + 1] - edges[i]) * align for i in range(n))
