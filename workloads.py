"""Seeded synthetic inputs for the ternary BitLinear mpGEMM.

This module only draws random numbers and describes layer shapes. It holds
none of the method's arithmetic (no quantization, ternarization, packing or
dot products), so both the CPU oracle and the HIP path can take their inputs
from it without sharing any of the computation they are compared on.

The pages evaluate trained ternary models (700M to 100B parameters) on
WikiText2 / HellaSwag / Winogrande (Bitnet.cpp reading notes, Part A §2.2).
Those weights and datasets are not available, so layers with the same shapes
and the value distributions below stand in for them.

Generator: numpy PCG64, seed = 1000*config + 10*projection + {0: weights,
1: activations}. Projection indices: q=0, k=1, v=2, o=3, gate=4, up=5, down=6.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")

# Absmean of N(0, 0.02): sigma * sqrt(2/pi). Used as the weight scale of the
# layers whose ternary values are drawn directly (no fp32 master weights).
GAMMA_DRAWN = float(np.float32(0.02 * math.sqrt(2.0 / math.pi)))


@dataclass(frozen=True)
class Proj:
    """One BitLinear projection: y[M][N] = W[N][K] applied to x[M][K]."""
    name: str
    index: int
    K: int
    N: int


@dataclass(frozen=True)
class LayerConfig:
    """A synthetic layer: its projections and how weights/activations are drawn.

    weights: "f32_normal" (fp32 N(0, 0.02), to be absmean-ternarized) or
             "ternary" (drawn directly with P(0) = p_zero, P(+1) = P(-1)).
    outlier_frac / outlier_scale: fraction of input channels (columns of x)
             multiplied by outlier_scale before rounding to bf16.
    """
    cid: int
    name: str
    projs: tuple
    Ms: tuple
    weights: str
    p_zero: float = 0.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    notes: str = ""

    @property
    def packed_bytes(self) -> int:
        return sum(p.N * p.K // 4 for p in self.projs)

    def ops(self, M: int) -> int:
        return sum(2 * M * p.N * p.K for p in self.projs)


def _layer(h: int, kv: int, ffn: int):
    shapes = [(h, h), (h, kv), (h, kv), (h, h), (h, ffn), (h, ffn), (ffn, h)]
    return tuple(Proj(n, i, K, N) for i, (n, (K, N)) in enumerate(zip(PROJ_NAMES, shapes)))


LAYERS = {
    1: LayerConfig(1, "single-1024x1024-decode", (Proj("single", 0, 1024, 1024),), (1,),
                   "f32_normal"),
    2: LayerConfig(2, "bitnet-2b-layer-decode", _layer(2560, 640, 6912), (1,),
                   "ternary", p_zero=0.40, outlier_frac=0.01, outlier_scale=20.0),
    3: LayerConfig(3, "bitnet-2b-layer-prefill-512", _layer(2560, 640, 6912), (512,),
                   "ternary", p_zero=0.40, outlier_frac=0.01, outlier_scale=20.0),
    4: LayerConfig(4, "7b-layer-decode", _layer(4096, 4096, 11008), (1, 4, 16),
                   "f32_normal"),
    5: LayerConfig(5, "100b-layer-prefill-2048", _layer(8192, 1024, 28672), (2048,),
                   "ternary", p_zero=1.0 / 3.0, outlier_frac=0.005, outlier_scale=50.0),
}


# The projections of a decoder layer that read one input and do not depend
# on each other, in layer order: one fused decode launch, or one grouped GEMM
# over one quantized input, per group.
LAYER_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def seed_for(cid: int, proj_index: int, what: int) -> int:
    """what: 0 = weights, 1 = activations."""
    return 1000 * cid + 10 * proj_index + what


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def weights_f32_normal(seed: int, N: int, K: int, sigma: float = 0.02) -> np.ndarray:
    """fp32 [N][K], i.i.d. N(0, sigma)."""
    return rng(seed).standard_normal((N, K), dtype=np.float32) * np.float32(sigma)


def ternary_drawn(seed: int, N: int, K: int, p_zero: float) -> np.ndarray:
    """int8 [N][K] in {-1, 0, +1}, P(0) = p_zero, P(+1) = P(-1) = (1 - p_zero)/2."""
    u = rng(seed).random((N, K), dtype=np.float32)
    p_pos = np.float32(p_zero + (1.0 - p_zero) / 2.0)
    out = np.where(u < np.float32(p_zero), 0, np.where(u < p_pos, 1, -1))
    return out.astype(np.int8)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return the uint16 bit patterns.

    Used only to produce bf16 inputs from random fp32 draws.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def outlier_channels(seed: int, K: int, frac: float) -> np.ndarray:
    """round(frac*K) input-channel indices taken from a seeded permutation."""
    n = int(round(frac * K))
    return np.sort(rng(seed + 7919).permutation(K)[:n])


def activations_bf16(seed: int, M: int, K: int, outlier_frac: float = 0.0,
                     outlier_scale: float = 1.0) -> np.ndarray:
    """bf16 bits [M][K]: N(0, 1), with a shared set of outlier columns scaled."""
    x = rng(seed).standard_normal((M, K), dtype=np.float32)
    if outlier_frac > 0.0:
        cols = outlier_channels(seed, K, outlier_frac)
        x[:, cols] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def norm_inputs(seed: int, M: int, K: int, outlier_frac: float = 0.0,
                outlier_scale: float = 1.0, residual_sigma: float = 4.0):
    """bf16 bits for the fused residual add + RMSNorm + quantize step:
    x [M][K] (a sublayer's output: N(0, 1) with the outlier columns scaled),
    r [M][K] (the residual stream: N(0, residual_sigma^2)) and the norm weight
    g [K] (1 + 0.1 * N(0, 1)). The pages give no norm weights; these stand in."""
    x = activations_bf16(seed, M, K, outlier_frac, outlier_scale)
    r = rng(seed + 104729).standard_normal((M, K), dtype=np.float32) * np.float32(residual_sigma)
    g = np.float32(1.0) + np.float32(0.1) * rng(seed + 1299709).standard_normal(K, dtype=np.float32)
    return x, f32_to_bf16_bits(r), f32_to_bf16_bits(g)


@dataclass
class ProjInputs:
    proj: Proj
    M: int
    x_bf16: np.ndarray                 # uint16 [M][K]
    w_f32: np.ndarray | None = None     # fp32 [N][K] (f32_normal configs)
    w_tern: np.ndarray | None = None    # int8 [N][K] (drawn ternary configs)
    gamma: float | None = None          # given scale for drawn ternary


def proj_inputs(cfg: LayerConfig, proj: Proj, M: int, *, with_acts: bool = True,
                p_zero_override: float | None = None) -> ProjInputs:
    """Seeded inputs of one projection at M tokens."""
    ws = seed_for(cfg.cid, proj.index, 0)
    xs = seed_for(cfg.cid, proj.index, 1)
    x = activations_bf16(xs, M, proj.K, cfg.outlier_frac, cfg.outlier_scale) if with_acts \
        else None
    if cfg.weights == "f32_normal" and p_zero_override is None:
        return ProjInputs(proj, M, x, w_f32=weights_f32_normal(ws, proj.N, proj.K))
    p0 = cfg.p_zero if p_zero_override is None else p_zero_override
    return ProjInputs(proj, M, x, w_tern=ternary_drawn(ws, proj.N, proj.K, p0),
                      gamma=GAMMA_DRAWN)


def small_case(seed: int, M: int, N: int, K: int, kind: str = "f32_normal",
               p_zero: float = 0.4, outlier_frac: float = 0.0, outlier_scale: float = 1.0):
    """Arbitrary-shape seeded case for parity tests: (x_bf16, w_f32 or w_tern)."""
    x = activations_bf16(2 * seed + 1, M, K, outlier_frac, outlier_scale)
    if kind == "f32_normal":
        return x, weights_f32_normal(2 * seed, N, K)
    return x, ternary_drawn(2 * seed, N, K, p_zero)


def int8_codes(seed: int, M: int, K: int, zero_rows=()) -> np.ndarray:
    """int8 [M][K] uniform in [-127, 127] (stand-in quantized activations)."""
    q = rng(seed).integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    for t in zero_rows:
        q[t] = 0
    return q


def positive_scales(seed: int, M: int, zero_rows=()) -> np.ndarray:
    """fp32 [M] per-token scales in [0.004, 0.06) (zero for the listed rows)."""
    d = (rng(seed).random(M, dtype=np.float32) * np.float32(0.056) + np.float32(0.004))
    d = d.astype(np.float32)
    for t in zero_rows:
        d[t] = 0
    return d
