"""Pins of the oracle's dithered rounding (golden-ratio Weyl dither).

The listing entry "Low-Discrepancy Dither for Quantized Recurrent State Caches"
names a deterministic golden-ratio Weyl dither in place of rounding.  The
oracle's reading: code = clamp(floor(S*inv + u)) with u the Weyl sequence
frac(i * (sqrt(5)-1)/2) in 32-bit fixed point, i = step*Dv*Dk + r*Dk + c.
These tests tie it to things other than its own formula:
  * the offsets it uses agree with frac(i * 0.6180339887...) computed here in
    50-digit decimal arithmetic (up to the fixed-point error, which is bounded),
    and exactly the top 23 bits of the 32-bit fixed-point rotation whose
    constant is derived here from sqrt(5);
  * over many steps the codes average to the exact value (dither is unbiased,
    and a low-discrepancy sequence gets there at rate ~log(T)/T);
  * integers are left unchanged, out-of-range values clamp, every code is
    floor(y) or floor(y) + 1.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import OracleConfig

getcontext().prec = 60
PHI_C = (Decimal(5).sqrt() - 1) / 2          # golden-ratio conjugate


def _cfg(dv=4, dk=64, step=0):
    return OracleConfig(batch=1, heads=1, dk=dk, dv=dv, bits=8, group=dk,
                        policy=oracle.POLICY_PERSISTENT, rounding=oracle.ROUND_DITHER,
                        delta=0, decay=oracle.DECAY_SCALAR, step=step)


def _step_constant(cfg, vrow, trace=None):
    """One step from S = 0 with unit scale, alpha = 1, beta = 1, k = 1: the
    fp32 state after the write is v_r in every column of row r, y = v_r."""
    st = oracle.zero_state(cfg)
    st.scales[:] = 1.0
    q = np.zeros((1, cfg.dk), np.float32)
    k = np.ones((1, cfg.dk), np.float32)
    v = np.asarray(vrow, np.float32).reshape(1, cfg.dv)
    oracle.step(cfg, st, q, k, v, np.ones(1, np.float32), np.ones(1, np.float32), trace=trace)
    return st.codes[0]


def test_offsets_follow_the_golden_ratio_rotation():
    fr = [0.5, 0.25, 0.75, 0.125]            # one threshold 1 - f per row
    checked = 0
    steps = list(range(6)) + [10_000, 25_000, 50_000]   # far positions magnify a wrong rotation
    for t in steps:
        cfg = _cfg(step=t)
        codes = _step_constant(cfg, fr)
        for r in range(cfg.dv):
            for c in range(cfg.dk):
                i = t * cfg.dv * cfg.dk + r * cfg.dk + c
                u = (i * PHI_C) % 1
                eps = Decimal(2) ** -23 + i * Decimal("1.2e-10")
                thr = 1 - Decimal(fr[r])
                # near the threshold, or near 0/1 where the fixed-point value wraps
                if min(abs(u - thr), u, 1 - u) <= eps:
                    continue
                assert codes[r, c] == (1 if u >= thr else 0), (t, r, c)
                checked += 1
    assert checked > len(steps) * 4 * 64 - 40


def test_offsets_are_the_fixed_point_rotation_on_a_23_bit_grid():
    """The reading's exact form: the rotation in 32-bit fixed point (the
    conjugate truncated to 32 fractional bits, derived here from sqrt(5), times
    i modulo 1), of which the top 23 bits are kept so that 1 + u is an fp32
    number in [1, 2).  Compared exactly, as rationals, at near and far
    positions; the offsets the oracle used come from its trace."""
    from fractions import Fraction
    from decimal import ROUND_FLOOR
    phi32 = int((PHI_C * 2 ** 32).to_integral_value(rounding=ROUND_FLOOR))
    for t in (0, 1, 3, 77, 50_000):
        cfg = _cfg(step=t)
        tr = {}
        _step_constant(cfg, [0.5, 0.25, 0.75, 0.125], trace=tr)
        u = tr["yp"][0]
        for r in range(cfg.dv):
            for c in range(cfg.dk):
                i = t * cfg.dv * cfg.dk + r * cfg.dk + c
                frac = Fraction((i * phi32) % 2 ** 32, 2 ** 32)
                want = Fraction((frac * 2 ** 23).__floor__(), 2 ** 23)
                assert Fraction(float(u[r, c])) == want, (t, r, c)
                assert np.float32(1.0 + u[r, c]) == 1.0 + u[r, c]     # 1 + u is an fp32 number


def test_dither_is_unbiased_over_steps():
    y = np.float32(0.3)                      # not a dyadic fraction
    T = 2000
    acc = np.zeros((4, 64))
    for t in range(T):
        codes = _step_constant(_cfg(step=t), [y, -y, 2.7, -5.1])
        acc += codes
    mean = acc / T
    want = np.array([float(y), -float(y), float(np.float32(2.7)), float(np.float32(-5.1))])
    assert np.all(np.abs(mean - want[:, None]) < 0.01)


def test_codes_are_floor_or_floor_plus_one_and_integers_stay():
    tr = {}
    codes = _step_constant(_cfg(step=7), [3.0, -2.0, 0.49, 200.0], trace=tr)
    assert np.all(codes[0] == 3) and np.all(codes[1] == -2)
    assert set(np.unique(codes[2])) <= {0, 1}
    assert np.all(codes[3] == 127)                      # clamped at qmax
    u = tr["yp"][0]
    assert np.all((u >= 0) & (u < 1))
    y = tr["y"][0]                                     # the exact S*inv
    assert np.all(y[0] == 3.0) and np.all(y[2] == np.float32(0.49))
    assert np.array_equal(codes[2], (y[2] + u[2] >= 1).astype(codes.dtype))


@pytest.mark.parametrize("bits", [4, 8])
def test_dither_differs_from_rne_only_by_one_step(bits):
    """On a random state the dithered code is within one of the nearest code."""
    rng = np.random.default_rng(3)
    base = dict(batch=2, heads=2, dk=64, dv=8, bits=bits, group=32,
                policy=oracle.POLICY_DYNAMIC, delta=1, decay=oracle.DECAY_SCALAR)
    S = rng.standard_normal((4, 8, 64)).astype(np.float32)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    k = rng.standard_normal((4, 64)).astype(np.float32)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((4, 8)).astype(np.float32)
    a = np.full(4, 0.9, np.float32)
    b = np.full(4, 0.5, np.float32)
    outs = {}
    for rnd in (oracle.ROUND_RNE, oracle.ROUND_DITHER):
        cfg = OracleConfig(rounding=rnd, step=11, **base)
        st = oracle.calibrate(cfg, S)
        tr = {}
        oracle.step(cfg, st, q, k, v, a, b, trace=tr)
        outs[rnd] = (st.codes.astype(int), tr)
    d = outs[oracle.ROUND_DITHER][0] - outs[oracle.ROUND_RNE][0]
    assert np.abs(d).max() <= 1 and np.abs(d).sum() > 0
    # the exact pre-rounding values are the same computation in both modes
    assert np.array_equal(outs[oracle.ROUND_DITHER][1]["y"], outs[oracle.ROUND_RNE][1]["y"])


def test_exact_integer_sums_round_up():
    """floor(y + u) when y + u is exactly an integer: y = 1 - u gives code 1."""
    cfg = _cfg(dv=1, step=7)
    tr = {}
    _step_constant(cfg, [0.5], trace=tr)
    u = tr["yp"][0, 0].astype(np.float64)            # this step's offsets of row 0
    k = (1.0 - u).astype(np.float32)                 # exact: u has 23 bits
    assert np.array_equal(k.astype(np.float64), 1.0 - u)
    st = oracle.zero_state(cfg)
    st.scales[:] = 1.0
    oracle.step(cfg, st, np.zeros((1, 64), np.float32), k[None, :], np.ones((1, 1), np.float32),
                np.ones(1, np.float32), np.ones(1, np.float32))
    assert np.all(st.codes[0, 0] == 1)
