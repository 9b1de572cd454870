"""Absmean ternarization of fp32 weights (oracle; test infrastructure only).

Sources:
  * "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading notes,
    Part A §1.1 and §2.3: weights take values in {-1, 0, +1} with one scale
    per tensor (BitNet b1.58, whose paper is the notes' first core reference,
    §6). The weight-quantization formula itself is missing from the notes'
    §4.1 text.
  * FairyFuse article, "三元量化方案": one scale alpha per layer, weight above
    +0.5 alpha -> +1, below -0.5 alpha -> -1, otherwise 0.

Reading taken: alpha = gamma = mean |W| over the whole matrix (BitNet b1.58's
absmean), computed from the exact sum of |w|:

  gamma = fl32( fl64(sum |w| exactly) / n ),   n = number of elements
  t     = fl32(0.5 * gamma)
  w_t   = +1 if w > t, -1 if w < -t, else 0    (strict: |w| == t -> 0)

The strict comparison equals RoundClip(w / gamma, -1, 1) with ties to even
(|w / gamma| == 1/2 -> 0). gamma == 0 only for an all-zero matrix, which
ternarizes to all zeros (no epsilon is added anywhere).
"""
from __future__ import annotations

import math

import numpy as np

THRESHOLD_FRACTION = 0.5


def _exact_abs_sum(w: np.ndarray) -> float:
    # math.fsum returns the correctly rounded (to fp64) value of the exact sum.
    return math.fsum(np.abs(w.astype(np.float64)).ravel().tolist())


def absmean_gamma(w: np.ndarray) -> np.float32:
    """gamma = fl32(fl64(exact sum |w|) / n) for an fp32 array of any shape."""
    w = np.asarray(w, dtype=np.float32)
    if w.size == 0:
        raise ValueError("empty weight matrix")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    s = _exact_abs_sum(w)
    return np.float32(s / float(w.size))


def _above(w: np.ndarray, t: np.float32) -> np.ndarray:
    return w > t


def ternarize(w: np.ndarray, gamma) -> np.ndarray:
    """fp32 weights + scale -> int8 {-1, 0, +1}, threshold t = fl32(0.5 * gamma)."""
    w = np.asarray(w, dtype=np.float32)
    t = np.float32(THRESHOLD_FRACTION) * np.float32(gamma)
    out = np.zeros(w.shape, dtype=np.int8)
    out[_above(w, t)] = 1
    out[_above(-w, t)] = -1
    return out


def ternarize_absmean(w: np.ndarray):
    """(ternary int8 [N][K], gamma fp32) for fp32 weights [N][K]."""
    g = absmean_gamma(w)
    return ternarize(w, g), g
