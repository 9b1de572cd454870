"""I2_S 2-bit packing of ternary weights (oracle; test infrastructure only).

Sources:
  * "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading notes,
    Part A §2.3 table: I2_S is an element-wise, multiply-add based format at
    2.0 bits per weight (one 2-bit code per weight, one scale per tensor).
  * FairyFuse article, "融合内核设计": ternary indices are stored bit-packed
    with the codes 00, 01, 10 standing for 0, +1, -1.

The code table is the FairyFuse one; the pages give no bit layout, so the
plainest one is taken: row-major [N][K/4] bytes, weight k of row n sits in
byte n*(K/4) + k//4 at bits 2*(k%4) .. 2*(k%4)+1 (first weight in the low
bits). Code 11 is never written; unpacking rejects it. K must be a multiple
of 4 (no padding rule exists).
"""
from __future__ import annotations

import numpy as np

CODE_ZERO = 0b00
CODE_POS = 0b01
CODE_NEG = 0b10
FIELDS_PER_BYTE = 4
FIELD_BITS = 2


def _field_shift(j: int) -> int:
    """Bit offset of the j-th weight (0..3) within its byte."""
    return FIELD_BITS * j


def pack_i2s(tern: np.ndarray) -> np.ndarray:
    """int8 {-1,0,+1} [N][K] -> uint8 [N][K/4]."""
    t = np.asarray(tern)
    if t.ndim != 2:
        raise ValueError("ternary weights must be 2-D [N][K]")
    N, K = t.shape
    if K % FIELDS_PER_BYTE:
        raise ValueError("K must be a multiple of 4")
    if not np.all((t == -1) | (t == 0) | (t == 1)):
        raise ValueError("weights must be in {-1, 0, +1}")
    codes = np.full(t.shape, CODE_ZERO, dtype=np.uint8)
    codes[t == 1] = CODE_POS
    codes[t == -1] = CODE_NEG
    c = codes.reshape(N, K // FIELDS_PER_BYTE, FIELDS_PER_BYTE)
    out = np.zeros((N, K // FIELDS_PER_BYTE), dtype=np.uint8)
    for j in range(FIELDS_PER_BYTE):
        out |= (c[:, :, j] << np.uint8(_field_shift(j))).astype(np.uint8)
    return out


def unpack_i2s(packed: np.ndarray, K: int) -> np.ndarray:
    """uint8 [N][K/4] -> int8 {-1,0,+1} [N][K]; raises on the unused code 11."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.ndim != 2 or p.shape[1] * FIELDS_PER_BYTE != K:
        raise ValueError("packed shape does not match K")
    N = p.shape[0]
    out = np.zeros((N, K // FIELDS_PER_BYTE, FIELDS_PER_BYTE), dtype=np.int8)
    for j in range(FIELDS_PER_BYTE):
        f = (p >> np.uint8(_field_shift(j))) & np.uint8(0b11)
        if np.any(f == 0b11):
            raise ValueError("invalid I2_S code 11")
        out[:, :, j] = np.where(f == CODE_POS, 1, np.where(f == CODE_NEG, -1, 0))
    return out.reshape(N, K)
