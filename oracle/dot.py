"""Exact integer contraction of int8 activations with ternary weights (oracle).

Test infrastructure only.

Sources:
  * "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading notes,
    Part A §2.3 / §4.1: I2_S is multiply-add based and lossless because no
    partial sum is re-quantized; Part B "方法公式化" states the lossless
    condition as ternary weights + int8 activations + no extra quantization.
  * bitnet.cpp how-to blog §1.2 and FairyFuse "融合内核设计": with weights in
    {-1, 0, +1} every product is an add, a subtract or nothing.

  acc[t][n] = sum_k q[t][k] * w[n][k]      (exact integer; int64 here)

|acc| <= 127*K, so int32 holds it exactly for K <= 16,909,320 and fp32 holds
it exactly while 127*K < 2**24 (K <= 132,104).
"""
from __future__ import annotations

import numpy as np

INT32_MAX = 2**31 - 1


def _check(q: np.ndarray, w: np.ndarray):
    if q.ndim != 2 or w.ndim != 2 or q.shape[1] != w.shape[1]:
        raise ValueError("q [M][K] and w [N][K] must share K")
    if 127 * q.shape[1] > INT32_MAX:
        raise ValueError("K too large for an exact int32 accumulator")


def _as_columns(w: np.ndarray) -> np.ndarray:
    """w [N][K] -> int64 [K][N], the right operand of q @ (.)."""
    return w.astype(np.int64).T


def mpgemm_acc(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """int8 q [M][K], int8 ternary w [N][K] -> int64 acc [M][N] (numpy integer matmul)."""
    q = np.asarray(q)
    w = np.asarray(w)
    _check(q, w)
    return q.astype(np.int64) @ _as_columns(w)


def mpgemm_acc_entries(q: np.ndarray, w: np.ndarray, rows, cols) -> np.ndarray:
    """acc at the listed (t, n) pairs only, each as its own int64 dot product."""
    q = np.asarray(q)
    w = np.asarray(w)
    _check(q, w)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    out = np.empty(rows.shape, dtype=np.int64)
    for i, (t, n) in enumerate(zip(rows.tolist(), cols.tolist())):
        out[i] = int(np.dot(q[t].astype(np.int64), w[n].astype(np.int64)))
    return out


def mpgemm_acc_f64blas(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Same sum through an fp64 BLAS matmul; exact because every partial sum is
    an integer of magnitude <= 127*K < 2**53. Returns int64."""
    q = np.asarray(q)
    w = np.asarray(w)
    _check(q, w)
    if 127 * q.shape[1] >= 2**53:
        raise ValueError("K too large for exact fp64 accumulation")
    r = q.astype(np.float64) @ w.astype(np.float64).T
    return r.astype(np.int64)
