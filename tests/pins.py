"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin raises AssertionError when the oracle disagrees with: a hand-worked
example (tests/golden/), a closed form, brute force on tiny inputs, exact
rational arithmetic, a second independent algorithm (lookup-table sums), or an
invariant of the mathematics. tests/test_oracle_pins.py runs them all;
tests/test_oracle_mutations.py plants plausible mistakes in the oracle and
checks that some pin fails for each.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle
import oracle.dequant
import oracle.dot
import oracle.i2s
import oracle.lut
import oracle.quant
import oracle.ternary

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_bits(values):
    """Exact fp32 values -> bf16 bit patterns (asserts exactness)."""
    a = np.asarray(values, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "fixture value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_bf16(r, shape, scale=1.0):
    x = (r.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32) & np.uint32(0xFFFF0000)   # truncate to a bf16 value
    return (u >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# quantize_act_absmax
# ----------------------------------------------------------------------------

def pin_quant_golden():
    for name in ("e1_quant_basic.json", "e2_quant_ties.json"):
        g = golden(name)
        q, d = oracle.quantize_act_absmax(bf16_bits(g["x"]))
        assert q.tolist() == g["q"], (name, q.tolist())
        assert d.view(np.uint32).tolist() == g["d_bits"], (name, d)


def pin_quant_special():
    # zero row; constant row; one-hot row; all-negative row
    x = np.array([[0.0] * 4, [3.0] * 4, [0.0, 0.0, -5.0, 0.0], [-2.0, -1.0, -0.5, -2.0]],
                 dtype=np.float32)
    q, d = oracle.quantize_act_absmax(bf16_bits(x))
    assert q[0].tolist() == [0, 0, 0, 0] and d[0] == 0
    assert q[1].tolist() == [127] * 4
    assert q[2].tolist() == [0, 0, -127, 0]
    # m = 2, s = 63.5: -2 -> -127, -1 -> -63.5 -> -64 (even), -0.5 -> -31.75 -> -32
    assert q[3].tolist() == [-127, -64, -32, -127], q[3].tolist()
    assert d[3] == np.float32(2) / np.float32(127)
    q0, d0 = oracle.quantize_act_absmax(np.zeros((0, 8), dtype=np.uint16))
    assert q0.shape == (0, 8) and d0.shape == (0,)


def pin_quant_invariants(seed=11):
    r = _rng(seed)
    for scale in (1.0, 1e-3, 37.0, 1e20):
        xb = _rand_bf16(r, (9, 67), scale)
        x = oracle.widen_bf16(xb).astype(np.float64)
        q, d = oracle.quantize_act_absmax(xb)
        m = np.max(np.abs(x), axis=1)
        assert np.all(np.abs(q.astype(np.int64)) <= 127)
        # the absmax element of every row maps to exactly +-127
        for t in range(x.shape[0]):
            hot = np.abs(x[t]) == m[t]
            assert np.all(np.abs(q[t][hot]) == 127)
        # rounding error bound against the exact real x*127/m
        err = np.abs(q - x * 127.0 / m[:, None])
        assert np.all(err <= 0.5 + 1e-4), err.max()
        # d is the multiplier that maps 127 back to m (within one fp32 rounding)
        assert np.all(np.abs(d.astype(np.float64) * 127.0 - m) <= m * 2.0**-23)
        # sign symmetry
        qn, dn = oracle.quantize_act_absmax(xb ^ np.uint16(0x8000))
        assert np.array_equal(qn, -q) and np.array_equal(dn, d)
        # power-of-two scaling: same codes, d scales exactly
        for e in (-3, 5):
            xs = (oracle.widen_bf16(xb) * np.float32(2.0**e)).astype(np.float32)
            qs, ds = oracle.quantize_act_absmax((xs.view(np.uint32) >> 16).astype(np.uint16))
            assert np.array_equal(qs, q)
            assert np.array_equal(ds, (d * np.float32(2.0**e)).astype(np.float32))
        # monotone within a row
        for t in range(x.shape[0]):
            o = np.argsort(x[t], kind="stable")
            assert np.all(np.diff(q[t][o].astype(np.int64)) >= 0)


def pin_quant_rejects():
    bad = np.array([[0x7F80, 0]], dtype=np.uint16)  # +inf
    try:
        oracle.quantize_act_absmax(bad)
    except ValueError:
        pass
    else:
        raise AssertionError("inf accepted")


def pin_quant_tensor_golden():
    g = golden("e8_quant_tensor.json")
    q, d = oracle.quantize_act_absmax_tensor(bf16_bits(g["x"]))
    assert q.tolist() == g["q"], q.tolist()
    assert d.view(np.uint32).tolist() == g["d_bits"], d
    qt, _ = oracle.quantize_act_absmax(bf16_bits(g["x"]))
    assert qt[0].tolist() == g["q_per_token_row0"]       # the modes differ on token 0


def pin_quant_tensor_reductions(seed=22):
    """Per-tensor equals per-token for one token and for any token holding
    the tensor's absmax; every token shares d; bounds and symmetries."""
    r = _rng(seed)
    for scale in (1.0, 3e-2, 5e3):
        xb = _rand_bf16(r, (7, 45), scale)
        x = oracle.widen_bf16(xb).astype(np.float64)
        q, d = oracle.quantize_act_absmax_tensor(xb)
        qt, dt = oracle.quantize_act_absmax(xb)
        m = np.max(np.abs(x))
        for t in range(x.shape[0]):
            q1, d1 = oracle.quantize_act_absmax_tensor(xb[t:t + 1])
            assert np.array_equal(q1, qt[t:t + 1]) and np.array_equal(d1, dt[t:t + 1])
            if np.max(np.abs(x[t])) == m:
                assert np.array_equal(q[t], qt[t]) and d[t] == dt[t]
        assert np.all(d == d[0]) and abs(float(d[0]) * 127.0 - m) <= m * 2.0**-23
        err = np.abs(q - x * 127.0 / m)
        assert np.all(err <= 0.5 + 1e-4), err.max()
        assert np.max(np.abs(q.astype(np.int64))) == 127
        qn, dn = oracle.quantize_act_absmax_tensor(xb ^ np.uint16(0x8000))
        assert np.array_equal(qn, -q) and np.array_equal(dn, d)
        # monotone over the whole tensor (one scale)
        o = np.argsort(x.ravel(), kind="stable")
        assert np.all(np.diff(q.ravel()[o].astype(np.int64)) >= 0)
    z, dz = oracle.quantize_act_absmax_tensor(np.zeros((3, 8), dtype=np.uint16))
    assert not z.any() and not dz.any()


# ----------------------------------------------------------------------------
# residual + RMSNorm + quantize
# ----------------------------------------------------------------------------

def pin_norm_golden():
    for c in golden("e9_rmsnorm_quant.json")["cases"]:
        r = None if c["r"] is None else bf16_bits([c["r"]])
        h, q, d = oracle.rmsnorm_quant(bf16_bits([c["x"]]), r, bf16_bits(c["g"]), c["eps"])
        assert h[0].tolist() == c["h_bits"], (c["derivation"], h)
        assert q[0].tolist() == c["q"], (c["derivation"], q)
        assert int(d.view(np.uint32)[0]) == c["d_bits"], (c["derivation"], d)


def pin_norm_zero_rows():
    """A zero row gives q = 0, d = 0 with or without eps; so does a row whose
    residual cancels x exactly; negative eps is rejected."""
    g = bf16_bits([1.0, 2.0, 0.5, 1.0])
    x = bf16_bits([[0.0, 0.0, 0.0, 0.0], [1.5, -2.0, 0.25, 3.0], [1.0, 1.0, 1.0, 1.0]])
    r = bf16_bits([[0.0, 0.0, 0.0, 0.0], [-1.5, 2.0, -0.25, -3.0], [0.0, 0.0, 0.0, 0.0]])
    for eps in (0.0, 1e-6):
        h, q, d = oracle.rmsnorm_quant(x, r, g, eps)
        assert not q[:2].any() and not d[:2].any()
        assert (h[1] & 0x7FFF == 0).all()
        if eps == 0.0:
            assert q[2].tolist() == [64, 127, 32, 64]    # y = [1, 2, 0.5, 1], ties to even
    try:
        oracle.rmsnorm_quant(x, r, g, -1e-6)
    except ValueError:
        pass
    else:
        raise AssertionError("negative eps accepted")


def _ms_by_mantissas(hb):
    """sum h^2 / K from integer significands and exponents (exact rational)."""
    from fractions import Fraction
    total = Fraction(0)
    for b in np.asarray(hb, dtype=np.uint16).tolist():
        e, m = (b >> 7) & 0xFF, b & 0x7F
        sig, ex = (m, -133) if e == 0 else (m | 0x80, e - 134)
        total += Fraction(sig * sig) * (Fraction(2) ** (2 * ex))
    return total / len(hb)


def pin_norm_exact_ms(seed=23):
    """The oracle's mean square is the exact rational (checked from integer
    significands), and its fp32 rounding is the nearest fp32 value."""
    r = _rng(seed)
    xb = _rand_bf16(r, (5, 37), 3.0)
    rb = _rand_bf16(r, (5, 37), 0.5)
    g = _rand_bf16(r, (37,), 1.0)
    h, q, d, ms = oracle.rmsnorm_quant(xb, rb, g, 1e-5, return_ms=True)
    for t in range(5):
        exact = _ms_by_mantissas(h[t])
        assert ms[t] == exact
        f = oracle.round_fraction_to_f32(exact)
        lo, hi = np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))
        from fractions import Fraction
        assert abs(Fraction(float(f)) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(f)) - exact) <= abs(Fraction(float(hi)) - exact)


def pin_norm_invariants(seed=24):
    r = _rng(seed)
    K = 48
    xb = _rand_bf16(r, (6, K), 1.0)
    g = _rand_bf16(r, (K,), 1.0)
    h, q, d = oracle.rmsnorm_quant(xb, None, g, 0.0)
    assert np.array_equal(h, xb)
    # power-of-two scaling of x (eps = 0): identical codes and scales
    for e in (-4, 3):
        xs = (oracle.widen_bf16(xb) * np.float32(2.0**e)).astype(np.float32)
        hs, qs, ds = oracle.rmsnorm_quant((xs.view(np.uint32) >> 16).astype(np.uint16), None, g, 0.0)
        assert np.array_equal(qs, q) and np.array_equal(ds, d)
    # sign symmetry
    hn, qn, dn = oracle.rmsnorm_quant(xb ^ np.uint16(0x8000), None, g, 0.0)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)
    # a permutation of the features (with g) permutes the codes
    p = r.permutation(K)
    hp, qp, dp = oracle.rmsnorm_quant(xb[:, p], None, g[p], 0.0)
    assert np.array_equal(qp, q[:, p]) and np.array_equal(dp, d)
    # a zero residual leaves h = x
    h0, q0, d0 = oracle.rmsnorm_quant(xb, np.zeros_like(xb), g, 0.0)
    assert np.array_equal(h0, xb) and np.array_equal(q0, q)
    # rows whose mean square is a power of 4, g = 1, eps = 0: rinv is a power
    # of two, so the codes are the plain per-token quantizer's codes
    ones = bf16_bits(np.ones(4))
    rows = bf16_bits([[2.0, -2.0, 2.0, 2.0], [0.5, 0.25, -0.5, 0.5], [4.0, 0.0, 0.0, 0.0]])
    for t in range(3):
        hx, qx, dx = oracle.rmsnorm_quant(rows[t:t + 1], None, ones, 0.0)
        qa, _ = oracle.quantize_act_absmax(rows[t:t + 1])
        msr = _ms_by_mantissas(rows[t])
        if msr.numerator in (1, 4, 16) and msr.denominator in (1, 4, 16, 64):
            assert np.array_equal(qx, qa), (t, qx, qa)


def pin_norm_error_bound(seed=25):
    """y within the stated fp32 roundings of the exact x/rms*g, codes within
    0.5 of y*127/max|y|."""
    from fractions import Fraction
    r = _rng(seed)
    xb = _rand_bf16(r, (4, 64), 2.0)
    g = _rand_bf16(r, (64,), 1.0)
    h, q, d, ms = oracle.rmsnorm_quant(xb, None, g, 1e-6, return_ms=True)
    hx = oracle.widen_bf16(h).astype(np.float64)
    gx = oracle.widen_bf16(g).astype(np.float64)
    for t in range(4):
        y = hx[t] / np.sqrt(float(ms[t]) + 1e-6) * gx
        m = np.max(np.abs(y))
        err = np.abs(q[t] - y * 127.0 / m)
        assert np.all(err <= 0.5 + 127 * 2.0**-20), err.max()


# ----------------------------------------------------------------------------
# absmean gamma and ternarize
# ----------------------------------------------------------------------------

def pin_ternary_golden():
    for name in ("e3_ternary_strict.json", "e4_ternary_gamma.json"):
        g = golden(name)
        w = np.array(g["w"], dtype=np.float32)
        t, gamma = oracle.ternarize_absmean(w)
        assert np.float32(gamma).view(np.uint32) == g["gamma_bits"][0], (name, gamma)
        assert t.tolist() == g["tern"], (name, t.tolist())


def _gamma_fraction(w):
    s = sum((Fraction(float(v)) for v in np.abs(w.astype(np.float64)).ravel()), Fraction(0))
    return np.float32(float(s) / float(w.size))   # float(Fraction) rounds correctly


def pin_gamma_exact(seed=12):
    r = _rng(seed)
    cases = [
        r.standard_normal((7, 13)).astype(np.float32) * np.float32(0.02),
        # one huge value among many small ones: sequential or pairwise sums lose the ones
        np.array([2.0**60] + [1.0] * 1023 + [2.0**-20] * 64, dtype=np.float32),
        # tiny magnitudes (subnormal fp32) next to normal ones
        np.array([1e-45, 3e-45, 1.0, 2.0**-126, 2.0**-130, 0.1, 0.3], dtype=np.float32),
        # widely spread exponents
        (r.standard_normal(500) * np.exp2(r.integers(-60, 60, 500))).astype(np.float32),
    ]
    for w in cases:
        g = oracle.absmean_gamma(w)
        assert np.float32(g).view(np.uint32) == _gamma_fraction(w).view(np.uint32), (g, w[:4])


def _roundclip_rational(w, gamma):
    out = np.zeros(w.shape, dtype=np.int8)
    G = Fraction(float(gamma))
    for i, v in enumerate(w.ravel().tolist()):
        rq = round(Fraction(v) / G)          # Fraction rounding: ties to even
        out.flat[i] = max(-1, min(1, rq))
    return out


def pin_ternary_roundclip(seed=13):
    """The threshold form equals RoundClip(w / gamma, -1, 1) (ties to even),
    evaluated with exact rationals, including weights placed exactly at and one
    ulp around +-gamma/2."""
    r = _rng(seed)
    w = (r.standard_normal((6, 40)) * 0.02).astype(np.float32)
    g = oracle.absmean_gamma(w)
    half = np.float32(0.5) * np.float32(g)
    specials = [half, -half, np.nextafter(half, np.float32(1)), np.nextafter(half, np.float32(0)),
                -np.nextafter(half, np.float32(1)), -np.nextafter(half, np.float32(0)),
                np.float32(0), np.float32(-0.0), np.float32(3) * half, -np.float32(3) * half]
    w[0, :len(specials)] = np.array(specials, dtype=np.float32)
    t = oracle.ternarize(w, g)
    assert np.array_equal(t, _roundclip_rational(w, g))


def pin_ternary_invariants(seed=14):
    r = _rng(seed)
    w = (r.standard_normal((16, 64)) * 0.02).astype(np.float32)
    t, g = oracle.ternarize_absmean(w)
    perm = r.permutation(w.size)
    tp, gp = oracle.ternarize_absmean(w.ravel()[perm].reshape(w.shape))
    assert gp == g and np.array_equal(tp.ravel(), t.ravel()[perm])
    for e in (-7, 9):
        te, ge = oracle.ternarize_absmean((w * np.float32(2.0**e)).astype(np.float32))
        assert np.array_equal(te, t) and ge == np.float32(g * np.float32(2.0**e))
    tn, gn = oracle.ternarize_absmean(-w)
    assert np.array_equal(tn, -t) and gn == g
    tz, gz = oracle.ternarize_absmean(np.zeros((3, 8), dtype=np.float32))
    assert gz == 0 and not np.any(tz)


def pin_ternary_statistics(seed=15):
    """Closed forms for N(0, sigma): E|w| = sigma*sqrt(2/pi); P(|w| <= E|w|/2) =
    erf(1/(2*sqrt(pi))) ~= 0.3101."""
    w = (_rng(seed).standard_normal((512, 1024)) * 0.02).astype(np.float32)
    t, g = oracle.ternarize_absmean(w)
    assert abs(float(g) - 0.02 * math.sqrt(2 / math.pi)) < 2e-5
    p0 = float(np.mean(t == 0))
    assert abs(p0 - math.erf(1 / (2 * math.sqrt(math.pi)))) < 3e-3, p0
    assert abs(float(np.mean(t == 1)) - float(np.mean(t == -1))) < 4e-3


# ----------------------------------------------------------------------------
# I2_S pack / unpack
# ----------------------------------------------------------------------------

def pin_pack_golden():
    g = golden("e5_pack_bytes.json")
    for case in g["cases"]:
        t = np.array(case["tern"], dtype=np.int8)
        p = oracle.pack_i2s(t)
        assert p.tolist() == case["packed"], (case["derivation"][:20], p.tolist())
        assert np.array_equal(oracle.unpack_i2s(p, t.shape[1]), t)


def pin_pack_exhaustive():
    """All 81 ternary 4-tuples <-> 81 distinct bytes (K = 4); every byte with a
    field 11 is rejected; round trips for full and partial groups."""
    tuples = np.array(list(itertools.product((-1, 0, 1), repeat=4)), dtype=np.int8)
    p = oracle.pack_i2s(tuples)        # 81 rows of K = 4 -> one byte each
    assert p.shape == (81, 1)
    assert len(set(p.ravel().tolist())) == 81
    assert np.array_equal(oracle.unpack_i2s(p, 4), tuples)
    valid = set(p.ravel().tolist())
    for b in range(256):
        fields = [(b >> (2 * j)) & 3 for j in range(4)]
        try:
            oracle.unpack_i2s(np.array([[b]], dtype=np.uint8), 4)
            ok = True
        except ValueError:
            ok = False
        assert ok == (3 not in fields)
        assert ok == (b in valid)
    r = _rng(22)
    for K in (8, 12, 16, 20, 28, 64, 260):
        t = r.integers(-1, 2, (7, K)).astype(np.int8)
        p = oracle.pack_i2s(t)
        assert p.shape == (7, K // 4)
        assert np.array_equal(oracle.unpack_i2s(p, K), t)


def pin_pack_layout():
    """One nonzero weight at a time: exactly one byte changes, and for full
    16-weight groups the 32-bit word shifted by 2*(k%16//4) and masked with
    0x03030303 holds the code in byte k%4 (the decode property the format is
    chosen for)."""
    N, K = 2, 36            # two full groups and a 4-weight tail
    for n in range(N):
        for k in range(K):
            for v, code in ((1, 0b01), (-1, 0b10)):
                t = np.zeros((N, K), dtype=np.int8)
                t[n, k] = v
                p = oracle.pack_i2s(t)
                nz = np.argwhere(p != 0)
                assert len(nz) == 1 and nz[0][0] == n
                if k < 32:
                    grp = k // 16
                    word = int.from_bytes(bytes(p[n, 4 * grp:4 * grp + 4].tolist()), "little")
                    i, j = (k % 16) // 4, k % 4
                    sel = (word >> (2 * i)) & 0x03030303
                    assert sel == code << (8 * j), (k, hex(word))
                else:
                    assert nz[0][1] == 8 and int(p[n, 8]) == code << (2 * (k - 32))


# ----------------------------------------------------------------------------
# exact contraction
# ----------------------------------------------------------------------------

def pin_dot_golden():
    g = golden("e6_dot.json")
    acc = oracle.mpgemm_acc(np.array(g["q"], dtype=np.int8), np.array(g["w"], dtype=np.int8))
    assert acc.tolist() == g["acc"], acc.tolist()


def pin_dot_bruteforce(seed=16):
    """All 81 ternary rows of K = 4 and a sample of K = 8 rows, against a
    pure-Python add/subtract loop."""
    r = _rng(seed)
    q = r.integers(-127, 128, (5, 4)).astype(np.int8)
    q[0] = [-127, 127, -127, 127]
    w = np.array(list(itertools.product((-1, 0, 1), repeat=4)), dtype=np.int8)
    acc = oracle.mpgemm_acc(q, w)
    for t in range(q.shape[0]):
        for n in range(w.shape[0]):
            s = 0
            for k in range(4):
                if w[n, k] == 1:
                    s += int(q[t, k])
                elif w[n, k] == -1:
                    s -= int(q[t, k])
            assert acc[t, n] == s
    q8 = r.integers(-127, 128, (3, 8)).astype(np.int8)
    w8 = r.integers(-1, 2, (200, 8)).astype(np.int8)
    acc8 = oracle.mpgemm_acc(q8, w8)
    for t in range(3):
        for n in range(200):
            assert acc8[t, n] == sum(int(q8[t, k]) * int(w8[n, k]) for k in range(8))
    # non-square shapes keep the [M][N] orientation
    assert oracle.mpgemm_acc(q8, w8).shape == (3, 200)


def pin_dot_lut(seed=17):
    """Lookup-table sums (g = 3 / g = 2 with mirror consolidation and the
    ThreeK/TwoK split) agree with the direct sum."""
    assert oracle.lut.class_counts() == (5, 14)
    r = _rng(seed)
    for K in (2, 3, 4, 5, 7, 8, 12, 16, 20, 64, 100):
        q = r.integers(-127, 128, (4, K)).astype(np.int8)
        w = r.integers(-1, 2, (9, K)).astype(np.int8)
        assert np.array_equal(oracle.lut_dot(q, w), oracle.mpgemm_acc(q, w)), K


def pin_dot_blas(seed=18):
    r = _rng(seed)
    q = r.integers(-127, 128, (17, 2560)).astype(np.int8)
    q[0] = 127
    w = r.integers(-1, 2, (33, 2560)).astype(np.int8)
    w[0] = 1
    assert np.array_equal(oracle.mpgemm_acc_f64blas(q, w), oracle.mpgemm_acc(q, w))
    rows = r.integers(0, 17, 40)
    cols = r.integers(0, 33, 40)
    full = oracle.mpgemm_acc(q, w)
    assert np.array_equal(oracle.mpgemm_acc_entries(q, w, rows, cols), full[rows, cols])


def pin_dot_invariants(seed=19):
    r = _rng(seed)
    K = 48
    q = r.integers(-127, 128, (6, K)).astype(np.int8)
    w = r.integers(-1, 2, (10, K)).astype(np.int8)
    acc = oracle.mpgemm_acc(q, w)
    p = r.permutation(K)
    assert np.array_equal(oracle.mpgemm_acc(q[:, p], w[:, p]), acc)
    ones = np.ones((2, K), dtype=np.int8)
    a1 = oracle.mpgemm_acc(q, ones)
    assert np.array_equal(a1[:, 0], q.astype(np.int64).sum(axis=1))
    assert np.array_equal(oracle.mpgemm_acc(q, -ones)[:, 1], -q.astype(np.int64).sum(axis=1))
    # additivity over disjoint supports
    mask = r.integers(0, 2, K).astype(bool)
    wa = np.where(mask, w, 0).astype(np.int8)
    wb = np.where(mask, 0, w).astype(np.int8)
    assert np.array_equal(oracle.mpgemm_acc(q, wa) + oracle.mpgemm_acc(q, wb), acc)


# ----------------------------------------------------------------------------
# dequant and bf16 rounding
# ----------------------------------------------------------------------------

def pin_dequant(seed=20):
    r = _rng(seed)
    acc = r.integers(-127 * 512, 127 * 512, (4, 9))
    acc[0, 0] = 0
    gamma = np.float32(0.0159577)
    d = (r.random(4) * 0.1).astype(np.float32)
    d[3] = 0
    y = oracle.dequant_f64(acc, gamma, d)
    y32 = oracle.dequant_f32(acc, gamma, d)
    G = Fraction(float(gamma))
    for t in range(4):
        for n in range(9):
            exact = Fraction(int(acc[t, n])) * G * Fraction(float(d[t]))
            if exact == 0:
                assert y[t, n] == 0 and y32[t, n] == 0
                continue
            assert abs(Fraction(float(y[t, n])) - exact) <= abs(exact) * Fraction(1, 2**52)
            assert abs(Fraction(float(y32[t, n])) - exact) <= abs(exact) * Fraction(25, 10**8)


def _bf16_nearest_rational(v: float) -> int:
    """Nearest bf16 of a normal-range double by exact rational search (ties to even)."""
    if v == 0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    m, e = math.frexp(a)                  # a = m * 2**e, 0.5 <= m < 1
    unit = Fraction(2) ** (e - 8)         # bf16 spacing in [2**(e-1), 2**e)
    k = Fraction(a) / unit                # 128 <= k < 256
    lo = math.floor(k)
    hi = lo + 1
    if k - lo < hi - k or (k - lo == hi - k and lo % 2 == 0):
        pick = lo
    else:
        pick = hi
    val = float(pick * unit)
    bits = int(np.float32(val).view(np.uint32)) >> 16
    return bits | (0x8000 if v < 0 else 0)


def pin_bf16_golden():
    g = golden("e7_bf16_ties.json")
    b = oracle.round_f64_to_bf16_bits(np.array(g["y"], dtype=np.float64))
    assert b.tolist() == g["bits"], [hex(v) for v in b.tolist()]


def pin_bf16_bruteforce(seed=21):
    r = _rng(seed)
    v = r.standard_normal(3000) * np.exp2(r.integers(-40, 40, 3000))
    # exact ties and near ties around random bf16 values
    base = oracle.bf16_bits_to_f64(r.integers(0x0100, 0x7F00, 200).astype(np.uint16))
    ulp = np.exp2(np.floor(np.log2(base)) - 7)
    v = np.concatenate([v, base + ulp / 2, base - ulp / 4, base + ulp / 2 * (1 + 2**-30),
                        -(base + ulp / 2), base])
    got = oracle.round_f64_to_bf16_bits(v)
    for x, b in zip(v.tolist(), got.tolist()):
        assert b == _bf16_nearest_rational(x), (x, hex(b))


# ----------------------------------------------------------------------------
# base-3 packing, five weights per byte
# ----------------------------------------------------------------------------

def pin_t3_golden():
    for c in golden("e10_t3_bytes.json")["cases"]:
        t = np.array(c["tern"], dtype=np.int8)
        b = oracle.pack_t3(t)
        assert b.tolist() == c["bytes"], c["derivation"]
        assert np.array_equal(oracle.unpack_t3(np.array(c["bytes"], np.uint8), c["K"]), t)


def pin_t3_exhaustive():
    """Every 5-tuple of ternary weights <-> one of 243 distinct bytes; the other
    13 byte values are rejected; the digits can be taken off the byte by
    repeated multiplication by 3 (y = 3x, digit = y >> 8, x = y mod 256)."""
    tuples = np.array(list(itertools.product((-1, 0, 1), repeat=5)), dtype=np.int8)
    w = np.zeros((243, 80), dtype=np.int8)
    for i in range(5):
        w[:, 16 * i] = tuples[:, i]                   # byte 0, planes 0..4
    b = oracle.pack_t3(w)
    assert len(set(b[:, 0].tolist())) == 243
    assert np.all(b[:, 1:] == b[0, 1:].min()) and b[0, 1] == 128    # zeros elsewhere
    valid = set(b[:, 0].tolist())
    for q in range(256):
        row = np.full((1, 64), 128, dtype=np.uint8)
        row[0, 0] = q
        if q in valid:
            got = oracle.unpack_t3(row, 80)
            assert tuple(got[0, 16 * np.arange(5)].tolist()) == tuple(
                tuples[b[:, 0].tolist().index(q)].tolist())
        else:
            try:
                oracle.unpack_t3(row, 80)
            except ValueError:
                continue
            raise AssertionError(f"byte {q} accepted")
    for t, q in zip(tuples.tolist(), b[:, 0].tolist()):
        x, digits = q, []
        for _ in range(5):
            y = 3 * x
            digits.append(y >> 8)
            x = y & 255
        assert [d - 1 for d in digits] == t, (t, q, digits)


def pin_t3_layout():
    """One nonzero weight at a time: exactly one byte changes, at 16u + (k%80)%16,
    by w * 3^(4-plane) in the base-3 value."""
    K = 400                                           # two row quanta, the second partial
    base = oracle.pack_t3(np.zeros((1, K), np.int8))
    assert base.shape == (1, 128) and np.all(base == 128)
    for k in (0, 15, 16, 63, 64, 79, 80, 159, 319, 320, 399):
        for w in (1, -1):
            t = np.zeros((1, K), np.int8)
            t[0, k] = w
            b = oracle.pack_t3(t)
            diff = np.nonzero(b[0] != base[0])[0].tolist()
            pos = 16 * (k // 80) + (k % 80) % 16
            assert diff == [pos], (k, diff)
            plane = (k % 80) // 16
            v = (243 * int(b[0, pos])) // 256
            assert v - 121 == w * 3 ** (4 - plane), (k, w, v)


def pin_t3_roundtrip_dot(seed=31):
    """unpack(pack(w)) = w; the contraction over the unpacked base-3 weights is
    the I2_S one; bytes per row = 64 * ceil(K / 320) (1.6 bits per weight when
    320 divides K); non-zero padding is rejected."""
    r = _rng(seed)
    for N, K in ((3, 16), (5, 320), (4, 336), (2, 2560), (3, 4160)):
        w = (r.integers(0, 3, (N, K)) - 1).astype(np.int8)
        b = oracle.pack_t3(w)
        assert b.shape == (N, 64 * -(-K // 320))
        assert np.array_equal(oracle.unpack_t3(b, K), w)
        q = r.integers(-127, 128, (2, K)).astype(np.int8)
        acc_t3 = oracle.mpgemm_acc(q, oracle.unpack_t3(b, K))
        acc_i2 = oracle.mpgemm_acc(q, oracle.unpack_i2s(oracle.pack_i2s(w), K))
        assert np.array_equal(acc_t3, acc_i2)
        assert np.array_equal(acc_t3, q.astype(np.int64) @ w.astype(np.int64).T)
    assert oracle.pack_t3(np.zeros((1, 3200), np.int8)).size * 8 / 3200 == 1.6
    bad = oracle.pack_t3(np.zeros((1, 16), np.int8))
    bad[0, 0] = 213                                    # plane 0 of byte 0 is real
    assert oracle.unpack_t3(bad, 16)[0, 0] == 1
    bad[0, 0] = 128 + 0                                # restore, then hit padding
    bad[0, 20] = 213                                   # byte 20: weight 84 > K
    try:
        oracle.unpack_t3(bad, 16)
    except ValueError:
        pass
    else:
        raise AssertionError("non-zero padding accepted")


def pin_token_sums():
    """Token sums of the codes: a hand-worked example, the closed form of a
    constant row, the contraction with an all-ones weight row (the pinned
    integer dot), and the offset-weight identity the GEMM relies on:
    sum_k (w+1) q = sum_k w q + S."""
    q = np.array([[1, -2, 3, -4], [127, -127, 0, 5], [0, 0, 0, 0]], dtype=np.int8)
    assert oracle.token_sums(q).tolist() == [-2, 5, 0]
    for c in (-127, -1, 0, 3, 127):
        assert oracle.token_sums(np.full((2, 4096), c, np.int8)).tolist() == [4096 * c] * 2
    r = _rng(32)
    q = r.integers(-127, 128, (7, 192)).astype(np.int8)
    w = r.integers(-1, 2, (5, 192)).astype(np.int8)
    s = oracle.token_sums(q)
    assert np.array_equal(oracle.mpgemm_acc(q, np.ones((1, 192), np.int8))[:, 0], s)
    acc1 = oracle.mpgemm_acc(q, (w + 1).astype(np.int8))
    assert np.array_equal(acc1 - s[:, None], oracle.mpgemm_acc(q, w))
    try:
        oracle.token_sums(q.astype(np.int16))
    except ValueError:
        pass
    else:
        raise AssertionError("non-int8 codes accepted")


ALL_PINS = [
    pin_quant_golden, pin_token_sums, pin_quant_special, pin_quant_invariants, pin_quant_rejects,
    pin_quant_tensor_golden, pin_quant_tensor_reductions,
    pin_t3_golden, pin_t3_exhaustive, pin_t3_layout, pin_t3_roundtrip_dot,
    pin_norm_golden, pin_norm_zero_rows, pin_norm_exact_ms, pin_norm_invariants, pin_norm_error_bound,
    pin_ternary_golden, pin_gamma_exact, pin_ternary_roundclip, pin_ternary_invariants,
    pin_ternary_statistics,
    pin_pack_golden, pin_pack_exhaustive, pin_pack_layout,
    pin_dot_golden, pin_dot_bruteforce, pin_dot_lut, pin_dot_blas, pin_dot_invariants,
    pin_dequant, pin_bf16_golden, pin_bf16_bruteforce,
]
