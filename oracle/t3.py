"""Base-3 packing of ternary weights, five weights per byte (1.6 bits per
weight) (oracle; test infrastructure only).

Sources: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
notes, Part A §2.3 (the mpGEMM format table: element-wise multiply-add
formats under 2 bits per weight, TQ1_0 at 1.69 and TL2 at 1.67 bits per
weight). A ternary weight has three values, so five of them fit one byte
(3^5 = 243 <= 256); the contraction over them is the same exact integer sum
as for I2_S.

Layout (the library's choice; the pages give no byte layout):
  * a row of K weights is padded with zero weights to a multiple of 320;
  * unit u of a row (weights 80u .. 80u+79) is 16 bytes at row offset 16u;
  * byte j (0..15) of a unit holds the five weights 80u + j + 16i, i = 0..4,
    so "plane" i of the unit's 16 bytes holds 16 consecutive weights;
  * the weights of a byte become digits d_i = w + 1 in {0, 1, 2} and the
    base-3 value v = sum_i d_i * 3^(4-i) in [0, 242] (d_0 most significant);
  * the byte stores q = ceil(256 v / 243): the byte read as the fraction
    q/256 starts with the base-3 digits of v, which is what lets a decoder
    take them off one at a time by multiplying by 3. v = floor(243 q / 256).
Bytes per row: 64 * ceil(K / 320). Of the 256 byte values, the 243 that
pack writes are valid; unpack rejects the others and non-zero padding.
"""
from __future__ import annotations

import numpy as np

UNIT = 80                # weights per 16-byte unit
UNIT_BYTES = 16
PLANES = 5               # weights per byte
ROW_QUANTUM = 320        # rows are padded to a multiple of this many weights
DIGIT_OFFSET = 1         # digit = weight + 1


def row_bytes(K: int) -> int:
    return 64 * ((K + ROW_QUANTUM - 1) // ROW_QUANTUM)


def _planes(w: np.ndarray) -> np.ndarray:
    """[N][Kp] -> [N][units][plane i][byte j]: weight 80u + j + 16i."""
    N, Kp = w.shape
    return w.reshape(N, Kp // UNIT, PLANES, UNIT_BYTES)


POW3 = np.array([3 ** (PLANES - 1 - i) for i in range(PLANES)], dtype=np.int64)   # 81 .. 1


def _encode(v):
    """Byte of base-3 value v: ceil(256 v / 243)."""
    return -((-256 * v) // 243)


def _decode(q):
    """Base-3 value of byte q: floor(243 q / 256)."""
    return (243 * q) // 256


def pack_t3(tern: np.ndarray) -> np.ndarray:
    """int8 {-1,0,+1} [N][K] -> uint8 [N][64*ceil(K/320)]."""
    t = np.asarray(tern)
    if t.ndim != 2:
        raise ValueError("ternary weights must be 2-D [N][K]")
    if not np.all((t == -1) | (t == 0) | (t == 1)):
        raise ValueError("weights must be in {-1, 0, +1}")
    N, K = t.shape
    Kp = row_bytes(K) // 64 * ROW_QUANTUM
    padded = np.zeros((N, Kp), dtype=np.int64)
    padded[:, :K] = t
    d = _planes(padded) + DIGIT_OFFSET                       # [N][U][5][16]
    v = np.einsum("nuij,i->nuj", d, POW3)                    # base-3 value per byte
    return _encode(v).reshape(N, -1).astype(np.uint8)


def unpack_t3(packed: np.ndarray, K: int) -> np.ndarray:
    """uint8 [N][64*ceil(K/320)] -> int8 [N][K]; rejects bytes pack never
    writes and padding that is not zero."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.ndim != 2 or p.shape[1] != row_bytes(K):
        raise ValueError("packed rows must hold 64*ceil(K/320) bytes")
    N = p.shape[0]
    q = p.astype(np.int64).reshape(N, -1, UNIT_BYTES)        # [N][U][16]
    v = _decode(q)
    if not np.array_equal(_encode(v), q):
        raise ValueError("a byte is not a valid base-3 encoding")
    d = (v[:, :, None, :] // POW3[None, None, :, None]) % 3  # [N][U][5][16]
    w = (d - DIGIT_OFFSET).astype(np.int8).reshape(N, -1)
    if np.any(w[:, K:] != 0):
        raise ValueError("padding weights must be zero")
    return w[:, :K].copy()
