"""Host-side model of the decode and GEMM kernels' global-memory addressing.

The kernels' loads are made unconditional (clamped) so the compiler can
overlap them; this model recomputes, for every block, wave, lane and
unrolled slot, the byte ranges those loads touch and checks they stay inside
the buffers, for the shapes the GPU tests and the benchmark use plus edge
cases. It mirrors the index arithmetic of k_decode_fast (gemv_i2s.hip) and
k_gemm_i2s (gemm_i2s.hip); it runs on the CPU and launches nothing.
"""
import itertools

import numpy as np
import pytest

WAVE = 64
LANES = np.arange(WAVE)
R_OF = LANES & 15
H_OF = LANES >> 4


def decode_fast_ranges(N, K, M, WK=4, U=None, ldx=None):
    """Yield (buffer, lo, hi) byte ranges of every load of one decode problem."""
    assert K % 64 == 0
    if K == 0:                      # routed to the zero-output kernel: no loads
        return
    ldx = K if ldx is None else ldx
    RB = K // 4
    nsteps = (K + 255) // 256
    length = (nsteps + WK - 1) // WK
    if U is None:
        U = 4 if length <= 4 else 8
    WR = 4 // WK
    blocks = (N + 16 * WR - 1) // (16 * WR)
    XREG, QREG = 8, 2
    for b, wv in itertools.product(range(blocks), range(4)):
        wr, wk = wv // WK, wv % WK
        n0 = (b * WR + wr) * 16
        ja = min(wk * length, nsteps)
        jb = min(ja + length, nsteps)
        klo, khi = min(ja * 256, K), min(jb * 256, K)
        kw = khi - klo
        rows = np.minimum(n0 + R_OF, N - 1)
        starts = list(range(ja, jb, 2 * U)) or [ja]
        for j in starts:
            for base in (j, j + U, j + 2 * U):
                for u in range(U):
                    step = max(min(base + u, jb - 1), 0)
                    off = np.minimum(step * 64 + 16 * H_OF, RB - 16)
                    lo = rows * RB + off
                    yield "packed", lo.min(), (lo + 16).max(), N * RB
        XF = (8 if length <= 4 else 16) if M == 1 else 0
        full_row = XF > 0 and K <= XF * 512            # whole bf16 row per wave (fused, M = 1)
        if full_row:
            nch8 = K // 8
            for u in range(XF):
                c = np.minimum(LANES + u * WAVE, nch8 - 1)
                lo = 16 * c
                yield "x", lo.min(), (lo + 16).max(), 2 * K
        cpt = kw // 4
        if M == 1 and not full_row and 0 < cpt <= XREG * WAVE:   # x range kept in registers
            for u in range(XREG):
                c = np.minimum(LANES + u * WAVE, cpt - 1)
                lo = 2 * (klo + 4 * c)
                yield "x", lo.min(), (lo + 8).max(), 2 * ((M - 1) * ldx + K)
        c16 = kw // 16
        if M == 1 and 0 < c16 <= QREG * WAVE:          # q chunks kept in registers
            for u in range(QREG):
                c = np.minimum(LANES + u * WAVE, c16 - 1)
                lo = klo + 16 * c
                yield "q", lo.min(), (lo + 16).max(), M * K


def gemm_ranges(N, K, M, RT=4, TT=8, WRW=2):
    """Yield byte ranges of every direct-to-LDS load of k_gemm_i2s."""
    BK = 128
    WTW = 4 // WRW
    BN, BM = WRW * RT * 16, WTW * TT * 16
    RB = K // 4
    nks = (K + BK - 1) // BK
    n_b_loads = BM * BK // (16 * 256)
    bchunk = 16 * ((LANES & 7) ^ ((LANES >> 3) & 7))
    for rb, tb in itertools.product(range((N + BN - 1) // BN), range((M + BM - 1) // BM)):
        n_blk, m_blk = rb * BN, tb * BM
        for ks, wv in itertools.product(range(nks), range(4)):
            kb = ks * BK
            boff = kb + bchunk
            boff = np.where(boff >= K, boff - 64, boff)
            for i in range(n_b_loads):
                t = (i * 4 + wv) * 8 + (LANES >> 3)
                tok = np.minimum(m_blk + t, M - 1)
                lo = tok * K + boff
                yield "q", lo.min(), (lo + 16).max(), M * K
            if wv * 32 < BN:
                row = wv * 32 + (LANES >> 1)
                n = np.minimum(n_blk + np.minimum(row, BN - 1), N - 1)
                aoff = kb // 4 + 16 * (LANES & 1)
                aoff = np.where(aoff >= RB, aoff - 16, aoff)
                lo = n * RB + aoff
                yield "packed", lo.min(), (lo + 16).max(), N * RB


DECODE_SHAPES = [(1, 64, 1), (5, 64, 1), (17, 128, 1), (640, 2560, 1), (2560, 6912, 1),
                 (100, 320, 4), (33, 64, 16), (2049, 256, 2), (5, 6912, 1), (300, 11008, 1),
                 (8, 64, 1), (1, 128, 1), (3, 0, 1), (130, 1024, 4), (7, 4096, 1)]


@pytest.mark.parametrize("N,K,M", DECODE_SHAPES, ids=[f"N{n}K{k}M{m}" for n, k, m in DECODE_SHAPES])
def test_decode_loads_in_bounds(N, K, M):
    for U in (4, 8):
        for buf, lo, hi, size in decode_fast_ranges(N, K, M, U=U):
            assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_decode_zero_k_launches_no_loads():
    assert list(decode_fast_ranges(5, 0, 3)) == []


GEMM_SHAPES = [(1, 64, 17), (130, 256, 17), (64, 2560, 64), (640, 320, 100), (257, 576, 129),
               (48, 6912, 65), (40, 256, 200), (7, 64, 20), (300, 192, 300)]


@pytest.mark.parametrize("N,K,M", GEMM_SHAPES, ids=[f"N{n}K{k}M{m}" for n, k, m in GEMM_SHAPES])
@pytest.mark.parametrize("tile", [(4, 8, 2), (2, 4, 2)], ids=["128x256", "64x128"])
def test_gemm_loads_in_bounds(N, K, M, tile):
    for buf, lo, hi, size in gemm_ranges(N, K, M, *tile):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_gemm_zero_k_issues_no_loads():
    assert list(gemm_ranges(7, 0, 20)) == []
