"""I2_S 2-bit packing of ternary weights (oracle; test infrastructure only).

Sources:
  * "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading notes,
    Part A §2.3 table: I2_S is an element-wise, multiply-add based format at
    2.0 bits per weight (one 2-bit code per weight, one scale per tensor).
  * FairyFuse article, "融合内核设计": ternary indices are stored bit-packed
    with the codes 00, 01, 10 standing for 0, +1, -1.

The code table is the FairyFuse one. The pages give no bit order; the
library's layout is:
  packed is uint8 [N][K/4]; each row is cut into groups of 16 weights
  (4 bytes), the last group of a row possibly shorter (4, 8 or 12 weights,
  i.e. b = 1, 2 or 3 bytes); inside a group of b bytes, weight o is stored in
  byte (o mod b) at bits 2*(o div b) .. 2*(o div b) + 1.
For a full group this puts weights 4i .. 4i+3 in field i of bytes 0..3, so a
shift by 2i and a mask of the group's 32-bit word gives them in byte order.
Code 11 is never written; unpacking rejects it. K must be a multiple of 4.
"""
from __future__ import annotations

import numpy as np

CODE_ZERO = 0b00
CODE_POS = 0b01
CODE_NEG = 0b10
WEIGHTS_PER_BYTE = 4
GROUP = 16          # weights per full group (one 32-bit word)
FIELD_BITS = 2


def _field_shift(i: int) -> int:
    """Bit offset of field i (0..3) within a byte."""
    return FIELD_BITS * i


def _groups(K: int):
    """(first weight, number of bytes b) of each group of a row of K weights."""
    out = []
    for k0 in range(0, K, GROUP):
        L = min(GROUP, K - k0)
        out.append((k0, L // WEIGHTS_PER_BYTE))
    return out


def pack_i2s(tern: np.ndarray) -> np.ndarray:
    """int8 {-1,0,+1} [N][K] -> uint8 [N][K/4]."""
    t = np.asarray(tern)
    if t.ndim != 2:
        raise ValueError("ternary weights must be 2-D [N][K]")
    N, K = t.shape
    if K % WEIGHTS_PER_BYTE:
        raise ValueError("K must be a multiple of 4")
    if not np.all((t == -1) | (t == 0) | (t == 1)):
        raise ValueError("weights must be in {-1, 0, +1}")
    codes = np.full(t.shape, CODE_ZERO, dtype=np.uint8)
    codes[t == 1] = CODE_POS
    codes[t == -1] = CODE_NEG
    out = np.zeros((N, K // WEIGHTS_PER_BYTE), dtype=np.uint8)
    for k0, b in _groups(K):
        g = codes[:, k0:k0 + 4 * b].reshape(N, 4, b)   # [row][field i][byte j], o = i*b + j
        byte0 = k0 // WEIGHTS_PER_BYTE
        for i in range(4):
            out[:, byte0:byte0 + b] |= (g[:, i, :] << np.uint8(_field_shift(i))).astype(np.uint8)
    return out


def unpack_i2s(packed: np.ndarray, K: int) -> np.ndarray:
    """uint8 [N][K/4] -> int8 {-1,0,+1} [N][K]; raises on the unused code 11."""
    p = np.asarray(packed, dtype=np.uint8)
    if K % WEIGHTS_PER_BYTE or p.ndim != 2 or p.shape[1] * WEIGHTS_PER_BYTE != K:
        raise ValueError("packed shape does not match K")
    N = p.shape[0]
    out = np.zeros((N, K), dtype=np.int8)
    for k0, b in _groups(K):
        byte0 = k0 // WEIGHTS_PER_BYTE
        for i in range(4):
            f = (p[:, byte0:byte0 + b] >> np.uint8(_field_shift(i))) & np.uint8(0b11)
            if np.any(f == 0b11):
                raise ValueError("invalid I2_S code 11")
            vals = np.where(f == CODE_POS, 1, np.where(f == CODE_NEG, -1, 0))
            out[:, k0 + i * b:k0 + (i + 1) * b] = vals
    return out
