"""Residual add + RMSNorm fused with absmax int8 quantization (oracle; test
infrastructure only).

Source: BinaryAI Engine forum post, "关键技术机制解析" §2: the residual add
and the RMS normalization run as one pass over the activations (half the
memory passes of running them apart). The quantizer that follows is the
per-token absmax int8 of the Bitnet.cpp reading notes, Part A §2.3 / §4.1.
The pages give no normalization formula; the readings taken (plain RMSNorm
with a per-feature weight, fp32 arithmetic with the roundings named here):

  h[t][k]  = bf16_rne(fl32(x[t][k] + r[t][k]))   (the new residual stream;
                                                  h = x when there is no r)
  ms_t     = fl32(sum_k h[t][k]^2 / K)            (exact sum, one rounding)
  rinv_t   = fl32(1 / fl32(sqrt(fl32(ms_t + eps))))
  y[t][k]  = fl32(fl32(h[t][k] * rinv_t) * g[k])  (g: bf16 norm weight)
  q, d     = per-token absmax int8 of y (as quantize_act_absmax, on fp32 y)

Degenerate rows (the pages are silent; the limit is taken): when
fl32(ms + eps) is zero (an all-zero row with eps = 0, or a mean square that
underflows fp32) the row normalizes to zero, so q = 0 and d = 0. eps must be
finite and >= 0; a mean square or a y that overflows fp32 is rejected.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .quant import QMAX, widen_bf16


_F32_MAX = Fraction(float(np.finfo(np.float32).max))


def _bf16_rne_from_f32(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def _f32_neighbours(fr: Fraction):
    """The two fp32 values around a positive rational (lo <= fr < hi)."""
    lo = np.float32(float(fr))
    while Fraction(float(lo)) > fr:
        lo = np.nextafter(lo, np.float32(0))
    hi = np.nextafter(lo, np.float32(np.inf))
    while Fraction(float(hi)) <= fr:
        lo, hi = hi, np.nextafter(hi, np.float32(np.inf))
    return lo, hi


def round_fraction_to_f32(fr: Fraction) -> np.float32:
    """Round a non-negative rational to fp32, to nearest with ties to even."""
    if fr == 0:
        return np.float32(0)
    lo, hi = _f32_neighbours(fr)
    if Fraction(float(lo)) == fr:
        return lo
    dl, dh = fr - Fraction(float(lo)), Fraction(float(hi)) - fr
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (int(lo.view(np.uint32)) & 1) == 0 else hi


def _exact_sum_squares(h: np.ndarray) -> Fraction:
    """sum of h^2 over one row, exactly (bf16 values are fp64-exact)."""
    return sum((Fraction(float(v)) ** 2 for v in h.astype(np.float64)), Fraction(0))


def _mean_square(h: np.ndarray) -> Fraction:
    return _exact_sum_squares(h) / h.shape[0]


def rmsnorm_quant(x_bits, r_bits, g_bits, eps: float, return_ms: bool = False):
    """x_bits, r_bits: uint16 bf16 [M][K] (r_bits may be None); g_bits: uint16
    bf16 [K]; eps: fp32 value. Returns (h_bits uint16 [M][K], q int8 [M][K],
    d fp32 [M]) (and the exact mean squares when return_ms)."""
    x = widen_bf16(x_bits)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M][K]")
    M, K = x.shape
    if r_bits is None:
        h_bits = np.asarray(x_bits, dtype=np.uint16).copy()
    else:
        s = (x + widen_bf16(r_bits)).astype(np.float32)            # fp32 add
        if not np.all(np.isfinite(s)):
            raise ValueError("non-finite residual sum")
        h_bits = _bf16_rne_from_f32(s)
    h = widen_bf16(h_bits)
    g = widen_bf16(g_bits)
    if not (np.all(np.isfinite(h)) and np.all(np.isfinite(g)) and np.isfinite(eps)):
        raise ValueError("non-finite input")
    if eps < 0:
        raise ValueError("eps must be >= 0")
    eps32 = np.float32(eps)
    q = np.zeros((M, K), dtype=np.int8)
    d = np.zeros(M, dtype=np.float32)
    mss = []
    for t in range(M):
        msf = _mean_square(h[t]) if K else Fraction(0)
        if msf > _F32_MAX:
            raise ValueError("mean square overflows fp32")
        mss.append(msf)
        ms = round_fraction_to_f32(msf)
        v = np.float32(ms + eps32)
        if v == 0:
            continue                                            # the row normalizes to zero
        rinv = np.float32(np.float32(1) / np.sqrt(v))           # fp32 sqrt, fp32 divide
        y = ((h[t] * rinv).astype(np.float32) * g).astype(np.float32)
        if not np.all(np.isfinite(y)):
            raise ValueError("normalized value overflows fp32")
        m = np.float32(np.max(np.abs(y))) if K else np.float32(0)
        if m == 0:
            continue
        sc = np.float32(QMAX) / m
        if not np.isfinite(sc):
            raise ValueError("absmax too small: 127/m overflows fp32")
        q[t] = np.clip(np.rint((y * sc).astype(np.float32)), -QMAX, QMAX).astype(np.int8)
        d[t] = m / np.float32(QMAX)
    if return_ms:
        return h_bits, q, d, mss
    return h_bits, q, d
