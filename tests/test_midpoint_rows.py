"""The midpoint-row generator (tests/midpoint_rows.py) against the oracle's
exact mean square: "tie" rows sit exactly on an fp32 rounding midpoint,
"above" and "below" rows lie strictly within 2^-70 (relative) of one, on the
stated side, at every magnitude the GPU tests use."""
from fractions import Fraction

import numpy as np
import pytest

import midpoint_rows as MR
import oracle


def _midpoint_offset(ms):
    f = oracle.round_fraction_to_f32(ms)
    lo, hi = np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))
    mids = [(Fraction(float(lo)) + Fraction(float(f))) / 2,
            (Fraction(float(f)) + Fraction(float(hi))) / 2]
    return min((ms - m for m in mids), key=abs)


@pytest.mark.parametrize("K", [64, 2560])
@pytest.mark.parametrize("scale", [0, -50, 40, -68])
def test_rows_are_what_they_claim(K, scale):
    rng = np.random.default_rng(1000 * K + scale + 100)
    for kind in ("tie", "above", "below"):
        for bg in (True, False):
            row = MR.midpoint_row(rng, K, kind, scale, bg)
            assert row is not None, (K, scale, kind, bg)
            ms = oracle.norm._mean_square(oracle.widen_bf16(row))
            off = _midpoint_offset(ms)
            if kind == "tie":
                assert off == 0
            else:
                assert 0 < abs(off) <= ms * Fraction(1, 2 ** 70)
                assert (off > 0) == (kind == "above")


def test_decompose_is_exact():
    t = Fraction(3, 7 * 2 ** 40) + Fraction(5)
    target = Fraction(int(t * 2 ** 60), 2 ** 60)
    bits = MR.decompose(target, 200)
    assert bits is not None
    assert sum(MR._bf16_value(b) ** 2 for b in bits) == target
