"""Host-side model of the decode and GEMM kernels' global-memory addressing.

The kernels' loads are made unconditional (clamped) so the compiler can
overlap them; this model recomputes, for every block, wave, lane and
unrolled slot, the byte ranges those loads touch and checks they stay inside
the buffers, for the shapes the GPU tests and the benchmark use plus edge
cases. It mirrors the index arithmetic of k_decode1 and k_gemvq (gemv_i2s.hip) and
k_gemm_i2s (gemm_i2s.hip); it runs on the CPU and launches nothing.
"""
import itertools

import numpy as np
import pytest

WAVE = 64
LANES = np.arange(WAVE)
R_OF = LANES & 15
H_OF = LANES >> 4


def steps_per_wave(K, wpb):
    return ((K + 255) // 256 + wpb - 1) // wpb


def decode1_config(K):
    """(WPB, XR, U, len) that launch_decode_group picks for a one-token group
    whose largest K is K: up to 8 steps a wave, one load batch of exactly the
    wave's steps."""
    len4 = steps_per_wave(K, 4)
    if len4 <= 4:
        return 4, (1 if len4 <= 2 else 2), max(len4, 1), len4
    len8 = steps_per_wave(K, 8)
    if len8 <= 4:
        return 8, 2, len8, len8
    if len8 <= 8:
        return 8, 4, len8, len8
    len16 = steps_per_wave(K, 16)
    assert len16 <= 16, "K above 65536 is rejected at the boundary"
    return (16, 4, len16, len16) if len16 <= 8 else (16, 8, 4, len16)


def gemvq_config(K, blocks32=0):
    """(WPB, U, RT) of launch_gemvq for a group whose largest K is K and whose
    problems hold blocks32 blocks of 32 rows in all."""
    two = blocks32 >= 256
    len4 = steps_per_wave(K, 4)
    if len4 <= 4:
        if two:
            return 4, (1 if len4 <= 2 else 2), 2
        return 4, max(len4, 1), 1
    len8 = steps_per_wave(K, 8)
    if len8 <= 4:
        return (8, 2, 2) if two else (8, len8, 1)
    return 16, 2, 1


def gemvq_ranges(N, K, M, group_kmax=None, blocks32=None):
    """Yield (buffer, lo, hi, size) of every global load of k_gemvq."""
    assert K % 64 == 0 and K >= 64 and 1 <= M <= 16
    WPB, U, RT = gemvq_config(K if group_kmax is None else group_kmax,
                              (N + 31) // 32 if blocks32 is None else blocks32)
    RB = K // 4
    nsteps = (K + 255) // 256
    length = (nsteps + WPB - 1) // WPB
    tok = np.minimum(R_OF, M - 1)
    for b, wk in itertools.product(range((N + 16 * RT - 1) // (16 * RT)), range(WPB)):
        ja = min(wk * length, nsteps)
        jb = min(ja + length, nsteps)
        starts = list(range(ja, jb, 2 * U)) or [ja]
        for j in starts:
            for base in (j, j + U, j + 2 * U):
                for u in range(U):
                    step = max(min(base + u, jb - 1), 0)
                    off = np.minimum(step * 64 + 16 * H_OF, RB - 16)
                    for rt in range(RT):
                        rows = np.minimum(b * 16 * RT + 16 * rt + R_OF, N - 1)
                        lo = rows * RB + off
                        yield "packed", lo.min(), (lo + 16).max(), N * RB
                    kk = np.minimum(step * 256 + 64 * H_OF, K - 64)
                    for s in range(4):
                        lo = tok * K + kk + 16 * s
                        yield "q", lo.min(), (lo + 16).max(), M * K


def decode1_ranges(N, K, group_kmax=None):
    """Yield (buffer, lo, hi, size) of every global load and LDS access of
    k_decode1 for one problem (one token) of a group whose largest K is
    group_kmax, and check the launch covers this K."""
    assert K % 64 == 0 and K >= 64
    WPB, XR, U, len_max = decode1_config(K if group_kmax is None else group_kmax)
    RB = K // 4
    nsteps = (K + 255) // 256
    length = (nsteps + WPB - 1) // WPB
    assert length <= len_max
    assert XR * WAVE * 8 >= length * 256          # the x chunks cover the part
    for b, wk in itertools.product(range((N + 15) // 16), range(WPB)):
        n0 = b * 16
        ja = min(wk * length, nsteps)
        jb = min(ja + length, nsteps)
        klo, khi = min(ja * 256, K), min(jb * 256, K)
        nch = (khi - klo) // 8
        cbase = klo // 8 if nch > 0 else 0
        clast = nch - 1 if nch > 0 else 0
        for u in range(XR):
            c = cbase + np.minimum(LANES + u * WAVE, clast)
            yield "x", (16 * c).min(), (16 * c + 16).max(), 2 * K
        rows = np.minimum(n0 + R_OF, N - 1)
        starts = list(range(ja, jb, 2 * U)) or [ja]
        for j in starts:
            for base in (j, j + U, j + 2 * U):
                for u in range(U):
                    step = max(min(base + u, jb - 1), 0)
                    off = np.minimum(step * 64 + 16 * H_OF, RB - 16)
                    lo = rows * RB + off
                    yield "packed", lo.min(), (lo + 16).max(), N * RB
        region = len_max * 256                     # the wave's LDS region
        if nch > 0:
            yield "lds", 0, 8 * nch, region
        yield "lds", 0, (jb - ja) * 256, region   # tail zeros and fragment reads


def gemm_ranges(N, K, M, RT=4, TT=8, WRW=2):
    """Yield byte ranges of every direct-to-LDS load of k_gemm_i2s."""
    BK = 128
    WTW = 4 // WRW
    BN, BM = WRW * RT * 16, WTW * TT * 16
    RB = K // 4
    nks = (K + BK - 1) // BK
    n_b_loads = BM * BK // (16 * 256)
    n_a_loads = -(-BN * (BK // 4) // (16 * 256))
    for rb, tb in itertools.product(range((N + BN - 1) // BN), range((M + BM - 1) // BM)):
        n_blk, m_blk = rb * BN, tb * BM
        for ks, wv in itertools.product(range(nks), range(4)):
            kb = ks * BK
            bchunk = 16 * ((LANES & 7) ^ swz(2 * (4 * (wv & 1) + (LANES >> 4))))
            boff = kb + bchunk
            boff = np.where(boff >= K, boff - 64, boff)
            for i in range(n_b_loads):
                t = (i * 4 + wv) * 8 + (LANES >> 3)
                tok = np.minimum(m_blk + t, M - 1)
                lo = tok * K + boff
                yield "q", lo.min(), (lo + 16).max(), M * K
            aoff = kb // 4 + 16 * ((LANES >> 4) & 1)
            aoff = np.where(aoff >= RB, aoff - 16, aoff)
            for i in range(n_a_loads):
                if (i * 4 + wv) * 32 >= BN:
                    continue
                row = (i * 4 + wv) * 32 + 16 * (LANES >> 5) + (LANES & 15)
                n = np.minimum(n_blk + np.minimum(row, BN - 1), N - 1)
                lo = n * RB + aoff
                yield "packed", lo.min(), (lo + 16).max(), N * RB


DECODE1_SHAPES = [(1, 64), (5, 64), (100, 320), (640, 2560), (2560, 2560), (6912, 2560),
                  (2560, 6912), (33, 16384), (17, 4160), (3, 1088), (2049, 256), (5, 6912),
                  (7, 11008), (3, 28672), (2, 32832), (2, 65536), (1, 40960)]


@pytest.mark.parametrize("N,K", DECODE1_SHAPES, ids=[f"N{n}K{k}" for n, k in DECODE1_SHAPES])
def test_decode1_loads_in_bounds(N, K):
    for buf, lo, hi, size in decode1_ranges(N, K):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_decode1_group_len_max():
    """In a group the LDS region is sized by the largest K; smaller problems
    stay inside it."""
    for K in (64, 320, 2560, 6912):
        for kmax in (7168, 28672, 65536):
            for buf, lo, hi, size in decode1_ranges(40, K, group_kmax=kmax):
                assert 0 <= lo and hi <= size, (buf, lo, hi, size)


GEMVQ_SHAPES = [(1, 64, 1), (5, 64, 16), (17, 128, 3), (640, 2560, 1), (2560, 6912, 4),
                (100, 320, 16), (33, 11008, 16), (2049, 256, 2), (5, 28672, 4),
                (300, 11008, 1), (7, 4160, 9), (3, 65536, 2)]


@pytest.mark.parametrize("N,K,M", GEMVQ_SHAPES, ids=[f"N{n}K{k}M{m}" for n, k, m in GEMVQ_SHAPES])
def test_gemvq_loads_in_bounds(N, K, M):
    for buf, lo, hi, size in gemvq_ranges(N, K, M):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_gemvq_group_kmax():
    for K in (64, 320, 4096):
        for buf, lo, hi, size in gemvq_ranges(20, K, 5, group_kmax=28672):
            assert 0 <= lo and hi <= size, (buf, lo, hi, size)


@pytest.mark.parametrize("N,K,M,blocks32", [(11008, 4096, 16, 688), (8193, 4096, 16, 257),
                                            (17, 4096, 8, 300), (4096, 2560, 16, 384),
                                            (33, 1024, 4, 256), (5000, 6912, 16, 300),
                                            (31, 64, 16, 256)])
def test_gemvq_two_row_tiles(N, K, M, blocks32):
    """Launches with at least 256 blocks of 32 rows give each wave two row
    tiles (also for a small problem inside a large group: its last block's
    second tile is clamped onto its last row)."""
    assert gemvq_config(K, blocks32)[2] == (2 if steps_per_wave(K, 8) <= 4 else 1)
    for buf, lo, hi, size in gemvq_ranges(N, K, M, blocks32=blocks32):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


GEMM_SHAPES = [(1, 64, 17), (130, 256, 17), (64, 2560, 64), (640, 320, 100), (257, 576, 129),
               (48, 6912, 65), (40, 256, 200), (7, 64, 20), (300, 192, 300)]


@pytest.mark.parametrize("N,K,M", GEMM_SHAPES, ids=[f"N{n}K{k}M{m}" for n, k, m in GEMM_SHAPES])
@pytest.mark.parametrize("tile", [(8, 4, 2), (4, 8, 2), (2, 4, 2), (1, 4, 2), (2, 2, 2)],
                         ids=["256x128", "128x256", "64x128", "32x128", "64x64"])
def test_gemm_loads_in_bounds(N, K, M, tile):
    for buf, lo, hi, size in gemm_ranges(N, K, M, *tile):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_gemm_zero_k_issues_no_loads():
    assert list(gemm_ranges(7, 0, 20)) == []


def gemm_lds_step(RT, TT, WRW):
    """Simulate one step's direct-to-LDS writes of k_gemm_i2s: returns dicts
    LDS byte -> (token, k byte) for activations and LDS byte -> (row, packed
    byte) for weights, plus the block geometry."""
    WTW = 4 // WRW
    BN, BM = WRW * RT * 16, WTW * TT * 16
    b_bytes = BM * 128
    n_b, n_a = BM * 128 // 4096, -(-BN * 32 // 4096)
    act, wts = {}, {}
    for wv in range(4):
        bchunk = 16 * ((LANES & 7) ^ swz(2 * (4 * (wv & 1) + (LANES >> 4))))
        for i in range(n_b):
            t = (i * 4 + wv) * 8 + (LANES >> 3)
            for l in range(WAVE):
                for b in range(16):
                    act[(i * 4 + wv) * 1024 + 16 * l + b] = (t[l], bchunk[l] + b)
        for i in range(n_a):
            if (i * 4 + wv) * 32 >= BN:
                continue
            row = (i * 4 + wv) * 32 + 16 * (LANES >> 5) + (LANES & 15)
            half = (LANES >> 4) & 1
            for l in range(WAVE):
                for b in range(16):
                    wts[b_bytes + (i * 4 + wv) * 1024 + 16 * l + b] = (row[l], 16 * half[l] + b)
    return act, wts, BN, BM, b_bytes


def swz(t):
    """Chunk swizzle of activation row t in k_gemm_i2s's LDS tile."""
    u = (t >> 1) & 7
    return u ^ ((((u >> 1) ^ (u >> 2)) & 1) << 1)


def lds_cycles(width):
    """Lane sets that one LDS cycle serves, as measured on gfx950 with the
    bank-conflict counter (pairs of active lanes reading one bank): a 64-bit
    read serves each 32-lane half at once, a 128-bit read each 32-lane half
    in two cycles split by the parity of lane bits 2, 3 and 4."""
    if width == 8:
        return [LANES[:32], LANES[32:]]
    par = ((LANES >> 2) ^ (LANES >> 3) ^ (LANES >> 4)) & 1
    return [LANES[(LANES >> 5 == half) & (par == p)] for half in (0, 1) for p in (0, 1)]


def banks_conflict_free(addrs, width):
    """64 banks of 4 bytes: the lanes of one cycle touch every bank at most once."""
    for lanes in lds_cycles(width):
        banks = [((addrs[l] + o) // 4) % 64 for l in lanes for o in range(0, width, 4)]
        if len(banks) != len(set(banks)):
            return False
    return True


def test_lds_cycle_model_matches_measurements():
    """The cycle model reproduces the probe outcomes it was fitted on: the
    plain (t/2) % 8 swizzle conflicts, so do 8-byte reads of 32-byte rows."""
    t = 16 + R_OF
    assert not banks_conflict_free(t * 128 + 16 * ((2 * H_OF) ^ ((t >> 1) & 7)), 16)
    assert not banks_conflict_free(t * 128 + 16 * ((2 * H_OF) ^ (t & 7)), 16)
    assert banks_conflict_free(LANES * 16, 16) and banks_conflict_free(LANES * 8, 8)
    assert not banks_conflict_free(R_OF * 32 + 8 * H_OF, 8)


@pytest.mark.parametrize("tile", [(4, 8, 2), (2, 4, 2), (1, 4, 2), (8, 4, 2), (2, 2, 2)])
def test_gemm_lds_fragments(tile):
    """Every MFMA fragment read of a step returns the intended operand bytes
    and every read instruction is free of bank conflicts."""
    RT, TT, WRW = tile
    act, wts, BN, BM, b_bytes = gemm_lds_step(RT, TT, WRW)
    for wv in range(4):
        wr, wt = wv % WRW, wv // WRW
        for s, tt in itertools.product(range(2), range(TT)):
            t = wt * TT * 16 + tt * 16 + R_OF
            p = (2 * H_OF + s) ^ swz(t)
            addr = t * 128 + 16 * p
            for l in range(WAVE):
                got = [act[addr[l] + b] for b in range(16)]
                want = [(t[l], 32 * H_OF[l] + 16 * s + b) for b in range(16)]
                assert got == want
            assert banks_conflict_free(addr, 16)
        for rt in range(RT):
            addr = b_bytes + (wr * RT + rt) * 512 + (H_OF >> 1) * 256 + R_OF * 16 + 8 * (H_OF & 1)
            for l in range(WAVE):
                got = [wts[addr[l] + b] for b in range(8)]
                want = [(wr * RT * 16 + rt * 16 + R_OF[l], 8 * H_OF[l] + b) for b in range(8)]
                assert got == want
            assert banks_conflict_free(addr, 8)


# ---- residual add + RMSNorm + quantize ------------------------------------

def rmsnorm_config(K, ldx):
    """(threads, chunks per thread) of the register-row kernel, or (256, 0)
    for the generic three-pass kernel (mirrors rmsnorm_quant_config)."""
    if K <= 0 or K % 8 or ldx % 8 or K > 32768:
        return 256, 0
    n = K // 8
    if n <= 4 * 256:
        return 256, -(-n // 256)
    return 1024, -(-n // 1024)


def rmsnorm_ranges(M, K, ldx):
    """Byte ranges touched per array: (lo, hi) over every thread and token."""
    nt, nc = rmsnorm_config(K, ldx)
    tid = np.arange(nt)
    row_lo, row_hi, qhi, ghi = [], [], [], []
    if nc:
        n = K // 8
        for i in range(nc):
            c = tid + i * nt
            load = np.minimum(c, n - 1)                       # clamped unconditional loads
            row_lo.append(16 * load.min())
            row_hi.append(16 * load.max() + 16)
            ghi.append(16 * load.max() + 16)
            st = c[c < n]
            if st.size:
                row_hi.append(16 * st.max() + 16)             # h_out store
                qhi.append(8 * st.max() + 8)
    else:
        c = np.arange(K // 4)
        row_lo.append(0)
        row_hi.append(8 * c.max() + 8)
        ghi.append(8 * c.max() + 8)
        qhi.append(4 * c.max() + 4)
    last = (M - 1) * ldx * 2
    return dict(x=(min(row_lo), last + max(row_hi)), g=(0, max(ghi)), q=(0, (M - 1) * K + max(qhi)),
                chunks=nc, threads=nt)


@pytest.mark.parametrize("K,ldx", [(8, 8), (40, 40), (2560, 2560), (2560, 2568), (4096, 4096),
                                   (6912, 6912), (8192, 8192), (8200, 8200), (11008, 11008),
                                   (28672, 28672), (32768, 32768), (36, 36), (2560, 2564),
                                   (32776, 32776), (40000, 40004), (4, 4)])
def test_rmsnorm_loads_in_bounds(K, ldx):
    M = 3
    r = rmsnorm_ranges(M, K, ldx)
    assert r["x"][0] >= 0 and r["x"][1] <= ((M - 1) * ldx + K) * 2      # x, r and h_out
    assert r["g"][1] <= 2 * K
    assert r["q"][1] <= M * K
    assert r["chunks"] <= 4 and r["threads"] in (256, 1024)
    if r["chunks"]:
        assert r["threads"] * r["chunks"] >= K // 8                     # every chunk covered


# ---- one-token decode of wide problems (whole-line weight loads) -----------

def wide_steps_per_wave(K, wpb):
    return ((K + 511) // 512 + wpb - 1) // wpb


def decode1w_config(K):
    """(WPB, XR, U, SINGLE, len) that launch_decode_group picks for a
    one-token group of wide problems whose largest K is K."""
    w4 = wide_steps_per_wave(K, 4)
    if w4 <= 4:
        w = max(w4, 1)
        return 4, w, w, True, w4
    w8 = wide_steps_per_wave(K, 8)
    if w8 <= 4:
        return 8, 4, 4, True, w8
    if w8 <= 8:
        return 8, 8, 2, False, w8
    w16 = wide_steps_per_wave(K, 16)
    assert w16 <= 8, "K above 65536 is rejected at the boundary"
    return 16, 8, 4, False, w16


C_OF = LANES >> 3
R8_OF = LANES & 7


def decode1w_ranges(N, K, group_kmax=None):
    """Yield (buffer, lo, hi, size) of every global load and LDS access of
    k_decode1w for one problem of a group whose largest K is group_kmax."""
    assert K % 64 == 0 and K >= 64
    WPB, XR, U, single, len_max = decode1w_config(K if group_kmax is None else group_kmax)
    RB = K // 4
    nsteps = (K + 511) // 512
    length = (nsteps + WPB - 1) // WPB
    assert length <= len_max
    assert XR * WAVE * 8 >= length * 512              # the x chunks cover the part
    if single:
        assert U >= length                            # one batch holds the whole run
    for b, wk in itertools.product(range((N + 15) // 16), range(WPB)):
        n0 = b * 16
        ja = min(wk * length, nsteps)
        jb = min(ja + length, nsteps)
        klo, khi = min(ja * 512, K), min(jb * 512, K)
        nch = (khi - klo) // 8
        cbase = klo // 8 if nch > 0 else 0
        clast = nch - 1 if nch > 0 else 0
        for u in range(XR):
            c = cbase + np.minimum(LANES + u * WAVE, clast)
            yield "x", (16 * c).min(), (16 * c + 16).max(), 2 * K
        rows = [np.minimum(n0 + R8_OF, N - 1), np.minimum(n0 + 8 + R8_OF, N - 1)]
        bases = [ja] if single else sorted({bb for j in (range(ja, jb, 2 * U) or [ja])
                                            for bb in (j, j + U, j + 2 * U)})
        for base in bases:
            for u in range(U):
                step = max(min(base + u, jb - 1), 0)
                off = np.minimum(step * 128 + 16 * C_OF, RB - 16)
                for r in rows:
                    lo = r * RB + off
                    yield "packed", lo.min(), (lo + 16).max(), N * RB
        region = len_max * 512
        if nch > 0:
            yield "lds", 0, 8 * nch, region
        if jb > ja:                                   # fragment reads of the last step
            hi = 64 * (2 * (H_OF.max()) + 1) + (jb - 1 - ja) * 512 + 48 + 16
            yield "lds", 0, hi, region


DECODE1W_SHAPES = [(8192, 64), (8200, 4160), (8192, 8192), (28672, 8192), (8192, 28672),
                   (8193, 11008), (9000, 512), (8192, 65536), (8192, 32768), (8208, 16448)]


@pytest.mark.parametrize("N,K", DECODE1W_SHAPES, ids=[f"N{n}K{k}" for n, k in DECODE1W_SHAPES])
def test_decode1w_loads_in_bounds(N, K):
    for buf, lo, hi, size in decode1w_ranges(N, K):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_decode1w_group_len_max():
    for K in (64, 512, 4160, 8192):
        for kmax in (8192, 28672, 65536):
            for buf, lo, hi, size in decode1w_ranges(40, K, group_kmax=kmax):
                assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_decode1w_mfma_pairing():
    """The chunk a lane loads and the activation chunk its MFMA column pairs
    with agree for the columns that are kept (0 for rows m < 8, 1 for m >= 8)."""
    for lane in range(WAVE):
        r8, c = lane & 7, lane >> 3
        m, h = lane & 15, lane >> 4                   # A operand position
        assert m == r8 + 8 * (c & 1) and h == c // 2
        col = 0 if m < 8 else 1                       # column kept for this row
        b_chunk = 2 * h + (col & 1)                   # activation chunk of that column
        assert b_chunk == c


# ---- base-3 GEMV ------------------------------------------------------------

def t3_config(K):
    """(WPB, U) of launch_gemv_t3."""
    steps = lambda wpb: ((K + 319) // 320 + wpb - 1) // wpb
    if steps(4) <= 2:
        return 4, max(steps(4), 1)
    if steps(8) <= 2:
        return 8, 2
    return 16, 2


def t3_ranges(N, K, M):
    WPB, U = t3_config(K)
    nsteps = (K + 319) // 320
    RBt = 64 * nsteps
    length = (nsteps + WPB - 1) // WPB
    for b, wk in itertools.product(range((N + 15) // 16), range(WPB)):
        ja = min(wk * length, nsteps)
        jb = min(ja + length, nsteps)
        rows = np.minimum(b * 16 + R_OF, N - 1)
        toks = np.minimum(R_OF, M - 1)
        starts = list(range(ja, jb, 2 * U)) or [ja]
        for j in starts:
            for base in (j, j + U, j + 2 * U):
                for u in range(U):
                    step = max(min(base + u, jb - 1), 0)
                    lo = rows * RBt + step * 64 + 16 * H_OF
                    yield "packed", lo.min(), (lo + 16).max(), N * RBt
                    for i in range(5):
                        kk = np.minimum(step * 320 + 80 * H_OF + 16 * i, K - 16)
                        lo = toks * K + kk
                        yield "q", lo.min(), (lo + 16).max(), M * K


@pytest.mark.parametrize("N,K,M", [(1, 16, 1), (17, 336, 3), (100, 2560, 16), (40, 4160, 2),
                                   (33, 6912, 1), (20, 28672, 4), (3, 65536, 16), (8, 1296, 1)])
def test_t3_loads_in_bounds(N, K, M):
    for buf, lo, hi, size in t3_ranges(N, K, M):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def decodet_config(K):
    """(WPB, XR, U, len) that launch_decode_group picks for a 2..4-token group
    (every ldx % 8 == 0, K <= 32768) whose largest K is K."""
    assert K <= 32768
    len4 = steps_per_wave(K, 4)
    if len4 <= 2:
        return 4, 1, 2, len4
    if len4 <= 4:
        return 4, 2, 4, len4
    len8 = steps_per_wave(K, 8)
    if len8 <= 4:
        return 8, 2, 4, len8
    if len8 <= 8:
        return 8, 4, 4, len8
    len16 = steps_per_wave(K, 16)
    assert len16 <= 8
    return 16, 4, 4, len16


MT = 4


def decodet_ranges(N, K, M, ldx, group_kmax=None):
    """Yield (buffer, lo, hi, size) of every global load and LDS access of
    k_decodeT (MT = 4 token slots) for one problem of an M-token group."""
    assert K % 64 == 0 and K >= 64 and 2 <= M <= MT and ldx >= K and ldx % 8 == 0
    WPB, XR, U, len_max = decodet_config(K if group_kmax is None else group_kmax)
    RB = K // 4
    nsteps = (K + 255) // 256
    length = (nsteps + WPB - 1) // WPB
    assert length <= len_max
    assert XR * WAVE * 8 >= length * 256
    tstride = len_max * 256 + 16
    assert tstride % 16 == 0
    lds_total = WPB * MT * tstride
    assert lds_total + (WPB - 1) * WAVE * 16 + MT * WPB * 4 <= 160 * 1024
    xsize = 2 * ((M - 1) * ldx + K)
    for b, wk in itertools.product(range((N + 15) // 16), range(WPB)):
        n0 = b * 16
        ja = min(wk * length, nsteps)
        jb = min(ja + length, nsteps)
        klo, khi = min(ja * 256, K), min(jb * 256, K)
        nch = (khi - klo) // 8
        cbase = klo // 8 if nch > 0 else 0
        clast = nch - 1 if nch > 0 else 0
        for t in range(MT):
            for u in range(XR):
                c = cbase + np.minimum(LANES + u * WAVE, clast)
                base = 2 * min(t, M - 1) * ldx
                assert base % 16 == 0
                yield "x", base + (16 * c).min(), base + (16 * c + 16).max(), xsize
        rows = np.minimum(n0 + R_OF, N - 1)
        starts = list(range(ja, jb, 2 * U)) or [ja]
        for j in starts:
            for base in (j, j + U, j + 2 * U):
                for u in range(U):
                    step = max(min(base + u, jb - 1), 0)
                    off = np.minimum(step * 64 + 16 * H_OF, RB - 16)
                    lo = rows * RB + off
                    yield "packed", lo.min(), (lo + 16).max(), N * RB
        wbase = wk * MT * tstride
        for t in range(MT):
            tb = wbase + t * tstride
            if nch > 0:
                yield "lds", tb, tb + 8 * nch, lds_total
            yield "lds", tb, tb + (jb - ja) * 256, lds_total
            # a token's region never reaches the next one
            assert (jb - ja) * 256 <= tstride - 16
        if b == 0 and nch > 0:
            for t in range(M):
                yield "q", t * K + klo, t * K + klo + 8 * nch, M * K


DECODET_SHAPES = [(1, 64, 2, 64), (5, 64, 4, 72), (100, 320, 3, 320), (2560, 2560, 4, 2560),
                  (6912, 2560, 2, 2568), (2560, 6912, 4, 6912), (33, 16384, 3, 16384),
                  (17, 4160, 4, 4168), (3, 1088, 2, 1088), (5, 11008, 4, 11008),
                  (3, 28672, 4, 28672), (2, 32768, 3, 32768), (4, 27648, 2, 27648)]


@pytest.mark.parametrize("N,K,M,ldx", DECODET_SHAPES,
                         ids=[f"N{n}K{k}M{m}ld{l}" for n, k, m, l in DECODET_SHAPES])
def test_decodet_loads_in_bounds(N, K, M, ldx):
    for buf, lo, hi, size in decodet_ranges(N, K, M, ldx):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_decodet_group_len_max():
    for K in (64, 320, 2560, 6912):
        for kmax in (7168, 28672, 32768):
            for buf, lo, hi, size in decodet_ranges(20, K, 4, K, group_kmax=kmax):
                assert 0 <= lo and hi <= size, (buf, lo, hi, size)


# ---- one-token fused decode over base-3 weights ----------------------------

def t3_segs_per_wave(K, wpb):
    nseg = ((K + 319) // 320 + 1) // 2
    return (nseg + wpb - 1) // wpb


def decode1_t3_config(K):
    """(WPB, XR, U, SINGLE, len) that launch_decode_group_t3 picks at M == 1."""
    w4 = t3_segs_per_wave(K, 4)
    if w4 <= 1:
        return 4, 2, 1, True, w4
    if w4 == 2:
        return 4, 3, 2, True, w4
    if w4 <= 4:
        return 4, 5, 4, True, w4
    w8 = t3_segs_per_wave(K, 8)
    if w8 <= 4:
        return 8, 5, 4, True, w8
    if w8 <= 8:
        return 8, 10, 4, False, w8
    w16 = t3_segs_per_wave(K, 16)
    return 16, 10, 4, False, w16


def decode1_t3_ranges(N, K, group_kmax=None):
    """Yield (buffer, lo, hi, size) of every global load and LDS access of
    k_decode1_t3 for one problem of a group whose largest K is group_kmax,
    and check that every LDS byte a fragment read covers was written."""
    assert K % 16 == 0 and K >= 16
    WPB, XR, U, single, len_max = decode1_t3_config(K if group_kmax is None else group_kmax)
    nsteps = (K + 319) // 320
    RBt = 64 * nsteps
    nseg = (nsteps + 1) // 2
    length = (nseg + WPB - 1) // WPB
    assert length <= len_max
    assert XR * WAVE >= length * 80                   # the x chunks cover the part
    if single:
        assert U >= length
    region = len_max * 640
    assert WPB * region + (WPB - 1) * 2 * WAVE * 16 + 4 * WPB <= 160 * 1024   # LDS per block
    for b, wk in itertools.product(range((N + 15) // 16), range(WPB)):
        n0 = b * 16
        ja = min(wk * length, nseg)
        jb = min(ja + length, nseg)
        klo, khi = min(ja * 640, K), min(jb * 640, K)
        assert (khi - klo) % 16 == 0
        nch = (khi - klo) // 8
        cbase = klo // 8 if nch > 0 else 0
        clast = nch - 1 if nch > 0 else 0
        for u in range(XR):
            c = cbase + np.minimum(LANES + u * WAVE, clast)
            yield "x", (16 * c).min(), (16 * c + 16).max(), 2 * K
        rows = [np.minimum(n0 + R8_OF, N - 1), np.minimum(n0 + 8 + R8_OF, N - 1)]
        bases = [ja] if single else sorted({bb for j in (range(ja, jb, 2 * U) or [ja])
                                            for bb in (j, j + U, j + 2 * U)})
        for base in bases:
            for u in range(U):
                seg = max(min(base + u, jb - 1), 0)
                off = np.minimum(seg * 128 + 16 * C_OF, RBt - 16)
                for r in rows:
                    lo = r * RBt + off
                    yield "packed", lo.min(), (lo + 16).max(), N * RBt
        written = np.zeros(region, bool)
        written[:8 * nch] = True                       # codes
        zb = np.arange(khi - klo, (jb - ja) * 640, 16)
        for z in zb:
            written[z:z + 16] = True                   # zeros past K
        if nch > 0:
            yield "lds", 0, 8 * nch, region
        if len(zb):
            yield "lds", int(zb.min()), int(zb.max()) + 16, region
        for seg in range(ja, jb):
            for p in range(5):
                lo = 80 * (2 * H_OF + (LANES & 1)) + (seg - ja) * 640 + 16 * p
                yield "lds", lo.min(), (lo + 16).max(), region
                for a in np.unique(lo):
                    assert written[a:a + 16].all(), (seg, p, a)


DECODE1_T3_SHAPES = [(16, 16), (17, 336), (2560, 2560), (640, 2560), (6912, 2560), (2560, 6912),
                     (1000, 4160), (28672, 8192), (8192, 28672), (40, 65536), (33, 61456),
                     (24, 12800), (8, 1296)]


@pytest.mark.parametrize("N,K", DECODE1_T3_SHAPES, ids=[f"N{n}K{k}" for n, k in DECODE1_T3_SHAPES])
def test_decode1_t3_loads_in_bounds(N, K):
    for buf, lo, hi, size in decode1_t3_ranges(min(N, 64), K):
        assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_decode1_t3_group_len_max():
    for K in (16, 336, 2560, 8192):
        for kmax in (2560, 8192, 28672, 65536):
            if kmax < K:                              # the group's largest K
                continue
            for buf, lo, hi, size in decode1_t3_ranges(20, K, group_kmax=kmax):
                assert 0 <= lo and hi <= size, (buf, lo, hi, size)


def test_decode1_t3_unit_pairing():
    """The unit a lane loads (c) is the unit whose codes its kept MFMA column
    reads: column n of k-group h reads unit 2h + (n & 1) of the segment."""
    for lane in range(WAVE):
        r8, c = lane & 7, lane >> 3
        m, h = lane & 15, lane >> 4
        assert m == r8 + 8 * (c & 1) and h == c // 2
        col = 0 if m < 8 else 1
        assert 2 * h + (col & 1) == c
    # row r of half i: D[r][0] (lane 16*(r//4), comp r%4) + D[8+r][1] (lane 33 + 16*(r//4))
    for r in range(8):
        lane0 = 16 * (r // 4)
        assert (lane0 & 15) == 0 and 4 * (lane0 >> 4) + r % 4 == r
        lane1 = lane0 + 33
        assert (lane1 & 15) == 1 and 4 * (lane1 >> 4) + r % 4 == 8 + r


# ---- the models follow the launchers --------------------------------------

def _dispatch_rules():
    """The one-token and 2..4-token launch choices of launch_decode_group,
    read from gemv_i2s.hip: {launcher: [(var, op, bound or None, template
    args, len var)]} in source order, and the step-count variables."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "mpgemm_token_absmax_amd", "csrc",
                            "gemv_i2s.hip")).read()
    body = src[src.index("hipError_t launch_decode_group(DecodeGroup"):]
    body = body[:body.index("\n}\n")]
    vars_ = {}
    for m in re.finditer(r"const int (\w+) = (wide_steps_per_wave|steps_per_wave)\(g, (\d+)\);",
                         body):
        vars_[m.group(1)] = (512 if m.group(2).startswith("wide") else 256, int(m.group(3)))
    rules = {}
    pat = (r"(?:if \((\w+) (<=|==) (\d+)\) )?return (launch_one_token_w|launch_one_token|"
           r"launch_tokens)<([^>]*)>\(g, (\w+), s\);")
    for m in re.finditer(pat, body):
        args = tuple(a.strip() for a in m.group(5).split(","))
        rules.setdefault(m.group(4), []).append(
            (m.group(1), m.group(2), int(m.group(3)) if m.group(3) else None, args, m.group(6)))
    return rules, vars_


def _pick(rules, vars_, K):
    vals = {v: ((K + sz - 1) // sz + w - 1) // w for v, (sz, w) in vars_.items()}
    for var, op, bound, args, lenvar in rules:
        if var is None or (op == "<=" and vals[var] <= bound) or (op == "==" and vals[var] == bound):
            return args, vals[lenvar]
    raise AssertionError(f"no launch for K = {K}")


def test_models_follow_the_launchers():
    """decode1_config, decode1w_config and decodet_config give the launch
    configuration that gemv_i2s.hip's dispatch picks, for every K."""
    rules, vars_ = _dispatch_rules()
    assert set(rules) == {"launch_one_token_w", "launch_one_token", "launch_tokens"}
    for K in range(64, 65536 + 1, 64):
        (wpb, rtw, xr, u), length = _pick(rules["launch_one_token"], vars_, K)
        assert rtw == "1"
        assert decode1_config(K) == (int(wpb), int(xr), int(u), length), K
        a, length = _pick(rules["launch_one_token_w"], vars_, K)
        assert decode1w_config(K) == (int(a[0]), int(a[1]), int(a[2]), a[3] == "true", length), K
        if K <= 32768:
            a, length = _pick(rules["launch_tokens"], vars_, K)
            assert decodet_config(K) == (int(a[0]), int(a[1]), int(a[2]), length), K
