"""Rows whose exact mean square sits on, or next to, an fp32 rounding midpoint.

Input generator for the RMSNorm tests (test infrastructure). A bf16 value
squared is a dyadic rational, so a target sum of squares T = K * m (m a
midpoint between two neighbouring fp32 values) can be written exactly as a
sum of bf16 squares by a greedy choice of the largest bf16 whose square fits
the remainder. Three kinds of row per midpoint:
  "tie"   sum of squares exactly K * m (the mean square is a tie);
  "above" K * m plus one square far below an fp64 ulp of the sum;
  "below" K * m minus such an amount.
In the last two an fp64 sum of the squares usually rounds to K * m exactly,
so only an exact sum rounds the mean square the right way. Everything here is
exact (Fractions); the rows are checked against the oracle, never against
each other.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _bf16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))


def _largest_bf16_square_at_most(t: Fraction) -> int:
    """Bits of the largest positive finite bf16 a with a*a <= t (t > 0), or 0."""
    a = float(t) ** 0.5
    bits = int(np.array([a], dtype=np.float32).view(np.uint32)[0]) >> 16
    bits = min(max(bits, 1), 0x7F7F)
    while bits > 0 and _bf16_value(bits) ** 2 > t:
        bits -= 1
    while bits < 0x7F7F and _bf16_value(bits + 1) ** 2 <= t:
        bits += 1
    return bits


def decompose(target: Fraction, max_terms: int):
    """bf16 bit patterns whose squares sum exactly to target, or None."""
    out = []
    t = target
    while t > 0:
        if len(out) >= max_terms:
            return None
        b = _largest_bf16_square_at_most(t)
        if b == 0:
            return None
        out.append(b)
        t -= _bf16_value(b) ** 2
    return out


def _f32_midpoint_above(f: np.float32) -> Fraction:
    nxt = np.nextafter(f, np.float32(np.inf))
    return (Fraction(float(f)) + Fraction(float(nxt))) / 2


def midpoint_row(rng: np.random.Generator, K: int, kind: str, scale_exp: int = 0,
                 background: bool = True):
    """One row of K bf16 bit patterns (uint16) of the given kind, or None when
    the greedy decomposition does not close within the row. The values are of
    magnitude about 2^scale_exp (the mean square about 4^scale_exp). With
    background, up to half the row is random N(0, 1/4) * 2^scale_exp values
    (truncated to bf16) and the decomposition covers the rest of the sum."""
    vals = np.zeros(K, dtype=np.uint16)
    s_bg = Fraction(0)
    n_bg = max(0, min(K // 2, K - 64)) if background else 0
    scale = Fraction(2) ** scale_exp
    if n_bg:
        bg = rng.standard_normal(n_bg) * 0.5 * 2.0 ** scale_exp
        bits = (bg.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # truncate
        vals[:n_bg] = bits
        s_bg = sum((_bf16_value(int(b) & 0x7FFF) ** 2 for b in bits), Fraction(0))
    # a midpoint above the background's own mean square
    lo = max(s_bg / K * Fraction(3, 2), scale * scale / 4)
    f = np.float32(float(lo * (1 + Fraction(int(rng.integers(0, 1 << 20)), 1 << 20))))
    m = _f32_midpoint_above(f)
    target = K * m - s_bg
    tiny = Fraction(1, 2 ** 80) * (K * m)
    if kind == "above":
        target += tiny
    elif kind == "below":
        target -= tiny
    elif kind != "tie":
        raise ValueError(kind)
    terms = decompose(target, K - n_bg)
    if terms is None:
        return None
    vals[n_bg:n_bg + len(terms)] = np.array(terms, dtype=np.uint16)
    signs = rng.integers(0, 2, K).astype(np.uint16) << 15
    vals = vals | np.where(vals != 0, signs, 0).astype(np.uint16)
    rng.shuffle(vals)
    return vals
