"""Per-token absmax int8 activation quantization (oracle; test infrastructure only).

Source: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading notes,
Part A §2.3 and §4.1: I2_S pairs the ternary weights with int8 activations
quantized with one scale over a whole vector (the notes contrast this with
per-block scales). One scale per token (row of x) is used here; at one token
it is the same as one scale for the whole activation tensor.

The pages give no formula. The readings taken (symmetric int8 with range
[-127, 127]; scale computed as a correctly rounded fp32 quotient; round half
to even; zero row -> zeros with scale 0):

  m_t  = max_k |x[t][k]|                (exact; order free)
  s_t  = fl32(127 / m_t)
  q    = clamp(round_half_even(fl32(x * s_t)), -127, 127)
  d_t  = fl32(m_t / 127)                (the dequantization multiplier)

quantize_act_absmax_tensor is the pages' literal setting for several tokens:
one scale over the whole activation tensor (same formulas with m = max over
every token and k; every token's d is the same value).

token_sums is not a quantity of the pages: it is the library's optional side
output of its quantizers, S_t = sum_k q[t][k], with which a contraction can
run on weights offset by one (sum_k (w+1) q = sum_k w q + S_t, exactly).
"""
from __future__ import annotations

import numpy as np

QMAX = 127  # symmetric int8 range [-QMAX, QMAX]


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values, exactly (bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round_half_even(v: np.ndarray) -> np.ndarray:
    return np.rint(v)


def _row_absmax(x: np.ndarray) -> np.ndarray:
    return np.max(np.abs(x), axis=1)


def quantize_act_absmax(x_bits: np.ndarray):
    """x_bits: uint16 bf16 patterns [M][K] -> (q int8 [M][K], d fp32 [M]).

    Raises ValueError for non-finite inputs and for rows whose absmax is so
    small that 127/m overflows fp32 (outside the method's domain).
    """
    x = widen_bf16(x_bits)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M][K]")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite activation")
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    d = np.zeros(M, dtype=np.float32)
    if M == 0 or K == 0:
        return q, d
    m = _row_absmax(x).astype(np.float32)
    nz = m > 0
    if not np.any(nz):
        return q, d
    s = np.float32(QMAX) / m[nz]                          # fp32 IEEE quotient
    if not np.all(np.isfinite(s)):
        raise ValueError("absmax too small: 127/m overflows fp32")
    v = (x[nz] * s[:, None]).astype(np.float32)           # fp32 product
    r = _round_half_even(v)
    q[nz] = np.clip(r, -QMAX, QMAX).astype(np.int8)
    d[nz] = m[nz] / np.float32(QMAX)                      # fp32 IEEE quotient
    return q, d


def _tensor_absmax(x: np.ndarray) -> np.float32:
    return np.float32(np.max(np.abs(x)))


def quantize_act_absmax_tensor(x_bits: np.ndarray):
    """One scale for the whole activation tensor ([BN] Part A 2.3 and 4.1:
    int8 activations with one per-tensor scale).

      m = max_{t,k} |x[t][k]|,  s = fl32(127 / m),
      q = clamp(round_half_even(fl32(x * s)), -127, 127),  d[t] = fl32(m / 127) for every t.

    x_bits: uint16 bf16 patterns [M][K] -> (q int8 [M][K], d fp32 [M]).
    Same domain as quantize_act_absmax.
    """
    x = widen_bf16(x_bits)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M][K]")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite activation")
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    d = np.zeros(M, dtype=np.float32)
    if M == 0 or K == 0:
        return q, d
    m = _tensor_absmax(x)
    if m == 0:
        return q, d
    s = np.float32(QMAX) / m                              # fp32 IEEE quotient
    if not np.isfinite(s):
        raise ValueError("absmax too small: 127/m overflows fp32")
    v = (x * s).astype(np.float32)                        # fp32 product
    q[:] = np.clip(_round_half_even(v), -QMAX, QMAX).astype(np.int8)
    d[:] = m / np.float32(QMAX)                           # fp32 IEEE quotient
    return q, d


def _row_total(q64: np.ndarray) -> np.ndarray:
    return q64.sum(axis=1)


def token_sums(q: np.ndarray) -> np.ndarray:
    """int8 codes [M][K] -> int64 [M]: S_t = sum_k q[t][k] (exact)."""
    q = np.asarray(q)
    if q.ndim != 2 or q.dtype != np.int8:
        raise ValueError("codes must be int8 [M][K]")
    return _row_total(q.astype(np.int64))
