"""The prefill's group scale fl(m / qmax) by a product and one corrective fma.

The prefill kernel forms a dynamic group scale s = fl(m / qmax) (qmax = 7 for
INT4 states, 127 for INT8) without a division instruction sequence:
q = fl(m * c) with c = fl(1 / qmax), the exact residual r = fma(-q, qmax, m),
then s = fma(r, c, q).  Its codes are only bit-exact with the oracle, which
divides, if that equals the IEEE quotient for every finite m >= 0.

This test emulates the three roundings exactly on the host and compares them
with numpy's IEEE float32 division, for every mantissa at the lowest
exponents (subnormal and near-subnormal quotients and residuals), at exponent
0 and at the top of the range.  Between those, every operation scales by the
same power of two, so the comparison carries over; the same sweep over every
finite float (all 255 exponents, both divisors) finds no difference either.
Infinite m is outside the identity (it gives NaN) and takes IEEE division in
the kernel.
"""
import numpy as np
import pytest


def _rn32(x):
    return x.astype(np.float32)


def fma_division(m32, qmax):
    """s = fma(fma(-q, qmax, m), c, q), q = fl(m c), with exact emulation of each rounding."""
    c = np.float32(1.0) / np.float32(qmax)
    m = m32.astype(np.float64)
    q = _rn32(m * np.float64(c))                    # exact product, one rounding
    r = _rn32(m - q.astype(np.float64) * qmax)      # exact in float64, one rounding
    t = r.astype(np.float64) * np.float64(c)        # exact (48 significant bits)
    a = q.astype(np.float64)
    s = a + t                                       # Knuth's two-sum: s + e = a + t exactly
    bp = s - a
    e = (a - (s - bp)) + (t - bp)
    res = _rn32(s)
    # rounding s to float32 equals rounding s + e, unless s is a float32
    # midpoint and e breaks the tie
    rd = res.astype(np.float64)
    lo = np.where(rd > s, np.nextafter(res, np.float32(-np.inf)), res)
    hi = np.where(rd > s, res, np.nextafter(res, np.float32(np.inf)))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    ismid = s == mid
    res = np.where(ismid & (e > 0), hi, res)
    return np.where(ismid & (e < 0), lo, res)


@pytest.mark.parametrize("qmax", [7.0, 127.0])
@pytest.mark.parametrize("biased_exp", [0, 1, 2, 3, 127, 253, 254])
def test_equals_ieee_division(qmax, biased_exp):
    m = (np.arange(1 << 23, dtype=np.uint32) + np.uint32(biased_exp << 23)).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        got = fma_division(m, qmax)
    want = m / np.float32(qmax)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), m[bad][:4]


def test_the_emulation_sees_a_wrong_correction():
    """Without the corrective fma (s = q) the quotient is wrong on many mantissas."""
    m = (np.arange(1 << 20, dtype=np.uint32) + np.uint32(127 << 23)).view(np.float32)
    q = _rn32(m.astype(np.float64) * np.float64(np.float32(1.0) / np.float32(7.0)))
    assert (q.view(np.uint32) != (m / np.float32(7.0)).view(np.uint32)).sum() > 1000
