"""Element-wise lookup-table dot product (TL1/TL2 style); a cross-check only.

Test infrastructure only. This is not the hot path: it is a second, independent
way to reach the same exact integer sums as oracle.dot, used to pin that
module.

Source: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
notes, Part A §2.3 technical details and Part B key methods:
  * TL groups g activations (g = 2 for TL1, g = 3 for TL2), precomputes the
    partial sums for every ternary weight pattern of the group and looks them
    up with the weights' group index;
  * mirror consolidation: a pattern and its negation give opposite sums, so
    only half of the C**g patterns (C = 3) are stored, plus a sign;
  * for g = 3 this leaves 14 classes (13 nonzero + zero): a 4-bit index and a
    1-bit sign per 3 weights;
  * block-fitting split: K is cut into a part handled in groups of three
    ("ThreeK") and a remainder handled in groups of two ("TwoK").
Partial sums are kept as exact integers (the lossless "_1" variants).
"""
from __future__ import annotations

import itertools

import numpy as np


def _classes(g: int):
    """Representatives (zero pattern first, then patterns whose first nonzero is +1)
    and a map pattern -> (class index, sign)."""
    reps = [(0,) * g]
    for p in itertools.product((-1, 0, 1), repeat=g):
        nz = [v for v in p if v != 0]
        if nz and nz[0] == 1:
            reps.append(p)
    lookup = {}
    for c, r in enumerate(reps):
        lookup[r] = (c, 1)
        lookup[tuple(-v for v in r)] = (c, -1 if c else 1)
    return np.array(reps, dtype=np.int64), lookup


def split_three_two(K: int):
    """(ThreeK, TwoK) with ThreeK % 3 == 0, TwoK % 2 == 0, ThreeK + TwoK == K."""
    if K < 2 and K != 0:
        raise ValueError("K must be 0 or >= 2")
    three = 3 * (K // 3)
    while three >= 0 and (K - three) % 2:
        three -= 3
    if three < 0:
        raise ValueError("cannot split K")
    return three, K - three


def _lut_part(q: np.ndarray, w: np.ndarray, g: int) -> np.ndarray:
    M, K = q.shape
    N = w.shape[0]
    if K == 0:
        return np.zeros((M, N), dtype=np.int64)
    G = K // g
    reps, lookup = _classes(g)
    qa = q.astype(np.int64).reshape(M, G, g)
    # half table per token and group: H[t][grp][c] = sum_j reps[c][j] * q[t][grp*g+j]
    H = np.einsum("tgj,cj->tgc", qa, reps)
    cls = np.empty((N, G), dtype=np.int64)
    sgn = np.empty((N, G), dtype=np.int64)
    wg = w.reshape(N, G, g)
    for n in range(N):
        for grp in range(G):
            c, s = lookup[tuple(int(v) for v in wg[n, grp])]
            cls[n, grp] = c
            sgn[n, grp] = s
    acc = np.zeros((M, N), dtype=np.int64)
    gi = np.arange(G)
    for n in range(N):
        acc[:, n] = (H[:, gi, cls[n]] * sgn[n]).sum(axis=1)
    return acc


def lut_dot(q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """acc [M][N] via g=3 tables over ThreeK and g=2 tables over TwoK."""
    q = np.asarray(q)
    w = np.asarray(w)
    K = q.shape[1]
    three, two = split_three_two(K)
    acc = _lut_part(q[:, :three], w[:, :three], 3)
    acc += _lut_part(q[:, three:], w[:, three:], 2)
    return acc


def class_counts():
    """Number of stored classes (including zero) for g = 2 and g = 3."""
    return len(_classes(2)[0]), len(_classes(3)[0])
