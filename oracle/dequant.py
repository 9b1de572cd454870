"""Dequantization of the integer accumulator (oracle; test infrastructure only).

Source: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading notes,
Part A §2.3 (I2_S = int2 codes with one weight scale, int8 activations with
their own scale) and the BitNet b1.58 scheme the notes cite: the output of a
BitLinear is the integer sum rescaled by the weight scale and the activation
scale. The pages print no formula; the reading is

  y[t][n] = acc[t][n] * gamma * d_t      (d_t = absmax_t / 127)

computed here in fp64 (y_ref; acc, gamma and d are exact in fp64, so only the
final product rounds). The fp32 epilogue used by the library is defined as

  c_t = fl32(gamma * d_t);  y = fl32(fl32(acc) * c_t)

(acc is exact in fp32 for |acc| < 2**24), within 2 fp32 roundings of y_ref.
bf16 results are y rounded to nearest, ties to even.
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), dtype=np.float32)[0])
_F64_DROP = 45  # fp64 has 52 fraction bits, bf16 keeps 7


def _scale_product(gamma, d):
    """gamma * d_t in fp64 (both exact in fp64), one value per token."""
    return float(np.float32(gamma)) * np.asarray(d, dtype=np.float32).astype(np.float64)


def _tie_up(lo_odd: np.ndarray) -> np.ndarray:
    """At an exact tie, step up to hi when lo's last kept bit is odd (ties to even)."""
    return lo_odd


def dequant_f64(acc: np.ndarray, gamma, d: np.ndarray) -> np.ndarray:
    acc = np.asarray(acc)
    return acc.astype(np.float64) * _scale_product(gamma, d)[:, None]


def dequant_f32(acc: np.ndarray, gamma, d: np.ndarray) -> np.ndarray:
    acc = np.asarray(acc)
    if np.any(np.abs(acc) >= 2**24):
        raise ValueError("accumulator not exact in fp32")
    c = (np.float32(gamma) * np.asarray(d, dtype=np.float32)).astype(np.float32)
    return (acc.astype(np.float32) * c[:, None]).astype(np.float32)


def round_f64_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of each fp64 value, as uint16 bit patterns.

    The two bf16 neighbours of |y| are found by truncating the fp64 fraction
    to 7 bits (lo) and stepping one bf16 ulp up (hi); |y| - lo and hi - |y| are
    exact fp64 differences (each pair lies within a factor of two).
    Values in the bf16 subnormal range or beyond the bf16 maximum raise.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("non-finite value")
    neg = np.signbit(y)
    a = np.abs(y)
    if np.any((a > 0) & (a < 2.0**-126)):
        raise ValueError("bf16 subnormal range not covered")
    bits = a.view(np.uint64)
    lo_bits = bits & ~np.uint64((1 << _F64_DROP) - 1)
    hi_bits = lo_bits + np.uint64(1 << _F64_DROP)
    lo = lo_bits.view(np.float64)
    hi = hi_bits.view(np.float64)
    dlo = a - lo
    dhi = hi - a
    lo_odd = ((lo_bits >> np.uint64(_F64_DROP)) & np.uint64(1)).astype(bool)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & _tie_up(lo_odd))
    r = np.where(pick_hi, hi, lo)
    if np.any(r > _BF16_MAX):
        raise ValueError("bf16 overflow")
    out = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[neg] |= np.uint16(0x8000)
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
