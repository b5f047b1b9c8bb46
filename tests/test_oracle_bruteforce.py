"""Whole-step brute-force pins of the oracle.

(1) Exhaustive dyadic grids: every previous INT4 code matrix of a 2x2 state,
    with power-of-two scales and dyadic inputs, so that every fp32 operation
    of the step is exact and the oracle must reproduce the exact-rational
    matrix form of Eq. (1) (LinQuant summary, Theoretical Foundation) and the
    exhaustive nearest-code search bit for bit -- exact rounding ties included.
(2) Random fp32 inputs on small non-square states (Dv != Dk) for every policy,
    rounding, delta and decay: codes must equal the exact-rational brute force
    except where the exact pre-rounding value lies within a narrow band of a
    decision boundary (the oracle rounds intermediate values to fp32).
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import (OracleConfig, POLICY_DYNAMIC, POLICY_PERSISTENT, POLICY_YOKED, ROUND_RNE,
                    ROUND_BDR, DECAY_SCALAR, DECAY_DIAG)
from tests import exact_ref as X


# ------------------------------------------------------------------ exhaustive dyadic
def _nearest_even_vec(y, lo_ok=None, hi_ok=None):
    """Exhaustive nearest integer search over a window, ties to even (float64 exact)."""
    cands = np.arange(-64, 65, dtype=np.float64)
    d = np.abs(cands[None, :] - y[:, None])
    if lo_ok is not None:
        d = np.where(cands[None, :] >= lo_ok[:, None], d, np.inf)
    if hi_ok is not None:
        d = np.where(cands[None, :] <= hi_ok[:, None], d, np.inf)
    key = d + 1e-9 * (np.abs(cands[None, :]) % 2)      # prefer even on equal distance
    return cands[np.argmin(key, axis=1)]


GRID = [  # (alpha, beta, k, v, q) dyadic; scales are powers of two
    (1.0, 0.5, (0.5, -0.25), (0.75, -1.5), (1.0, 0.5)),
    (0.75, 1.0, (1.0, 0.0), (-0.5, 2.0), (0.25, -1.0)),
    (0.5, 0.25, (-0.75, 0.5), (3.0, 0.125), (-2.0, 1.0)),
    # designed ties: half-integer decayed codes with no write (delta = 0) ...
    (0.5, 1.0, (0.5, 0.5), (0.0, 0.0), (1.0, 1.0)),
    # ... and a write of exactly half a grid step in row 0, column 0
    (1.0, 1.0, (0.5, 0.0), (0.25, -0.5), (1.0, 1.0)),
]
TIE_POINTS = (3, 4)


@pytest.mark.parametrize("g", [1, 2])
@pytest.mark.parametrize("delta", [0, 1])
@pytest.mark.parametrize("rounding", [ROUND_RNE, ROUND_BDR])
@pytest.mark.parametrize("gi", range(len(GRID)))
def test_exhaustive_dyadic_2x2(g, delta, rounding, gi):
    alpha, beta, k, v, q = GRID[gi]
    allc = np.array(list(itertools.product(range(-7, 8), repeat=4)), np.int8).reshape(-1, 2, 2)
    n = allc.shape[0]
    cfg = OracleConfig(n, 1, 2, 2, 4, g, POLICY_PERSISTENT, rounding, delta, DECAY_SCALAR)
    scales = np.broadcast_to(np.array([[0.25, 0.5], [0.5, 1.0]])[:, :2 // g],
                             (n, 2, 2 // g)).astype(np.float32).copy()
    st = oracle.OracleState(codes=allc.copy(), scales=scales.copy())
    f = lambda x, shp: np.broadcast_to(np.array(x, np.float32), shp).copy()
    o, _ = oracle.step(cfg, st, f(q, (n, 2)), f(k, (n, 2)), f(v, (n, 2)), f(alpha, (n,)),
                       f(beta, (n,)))
    # exact matrix form in float64 (every value here is a short dyadic: exact)
    s_full = np.repeat(scales, g, axis=-1).astype(np.float64)
    Sprev = allc.astype(np.float64) * s_full
    K = np.array(k, np.float64)
    I = np.eye(2)
    Sp = Sprev * alpha
    S = Sp @ (I - delta * beta * np.outer(K, K)) + beta * np.outer(np.array(v), K)[None]
    np.testing.assert_array_equal(o, S @ np.array(q))
    y, yp = S / s_full, Sp / s_full
    u = Sp @ K
    w = beta * (np.array(v)[None, :] - delta * u)               # [n, 2]
    sig = np.sign(w)[:, :, None] * np.sign(K)[None, None, :]
    yf, ypf, sf = y.ravel(), yp.ravel(), sig.ravel()
    if rounding == ROUND_RNE:
        want = _nearest_even_vec(yf)
    else:
        want = np.where(sf > 0, _nearest_even_vec(yf, lo_ok=ypf),
                        np.where(sf < 0, _nearest_even_vec(yf, hi_ok=ypf), _nearest_even_vec(yf)))
    want = np.clip(want, -7, 7).reshape(n, 2, 2)
    ties = np.abs(y - np.floor(y)) == 0.5
    if gi in TIE_POINTS and (delta == 0 or gi == 4):
        assert ties.any()      # these grid points do exercise exact ties
    np.testing.assert_array_equal(st.codes, want)


# ------------------------------------------------------------------ random fp32, band
BAND = 1e-5


def _boundary_distance(y, yp, rounding):
    """Distance (code units) of the exact values to the nearest decision boundary."""
    d = abs(y - (np.floor(float(y)) + 0.5))
    d = min(d, abs(y - (np.floor(float(y)) - 0.5)), abs(y - (np.floor(float(y)) + 1.5)))
    if rounding == ROUND_BDR:
        d = min(d, abs(yp - round(float(yp))))
    return float(d)


CASES = [(pol, rnd, dl, dc, g)
         for pol in (POLICY_DYNAMIC, POLICY_PERSISTENT, POLICY_YOKED)
         for rnd in (ROUND_RNE, ROUND_BDR)
         for dl in (0, 1)
         for dc in (DECAY_SCALAR, DECAY_DIAG)
         for g in (2, 4)]


@pytest.mark.parametrize("pol,rnd,dl,dc,g", CASES)
def test_random_small_states_vs_exact(pol, rnd, dl, dc, g):
    rng = np.random.default_rng(1000 + len(CASES) * 0 + hash((pol, rnd, dl, dc, g)) % 1000)
    n, dv, dk, bits = 24, 3, 4, 4
    qm = 7
    cfg = OracleConfig(n, 1, dk, dv, bits, g, pol, rnd, dl, dc)
    codes = rng.integers(-qm, qm + 1, (n, dv, dk)).astype(np.int8)
    scales = np.exp(rng.uniform(-3, 1, (n, dv, dk // g))).astype(np.float32)
    ref = (codes * np.repeat(scales, g, -1) * rng.uniform(0.9, 1.1, (n, dv, dk))).astype(np.float32)
    st = oracle.OracleState(codes=codes.copy(), scales=scales.copy(),
                            ref=ref.copy() if pol == POLICY_YOKED else None)
    q = rng.standard_normal((n, dk)).astype(np.float32)
    k = rng.standard_normal((n, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = (rng.standard_normal((n, dv)) * 2).astype(np.float32)
    a = rng.uniform(0.5, 1.0, (n, dk) if dc == DECAY_DIAG else (n,)).astype(np.float32)
    b = rng.uniform(0.1, 1.5, (n,)).astype(np.float32)
    o, o_ref = oracle.step(cfg, st, q, k, v, a, b)
    excused = 0
    for h in range(n):
        ex = X.quantised_step_exact(
            dict(dv=dv, dk=dk, group=g, bits=bits, policy=pol, rounding=rnd, delta=dl, decay=dc),
            codes[h], scales[h], ref[h], q[h], k[h], v[h], a[h] if dc == DECAY_DIAG else a[h], b[h])
        ex_o = np.array([float(x) for x in ex["o"]])
        tol = 1e-6 * (np.abs(np.array([[float(x) for x in r] for r in ex["S"]])) @ np.abs(q[h])).max()
        np.testing.assert_allclose(o[h], ex_o, rtol=0, atol=tol + 1e-30)
        ex_s = np.array([[float(x) for x in r] for r in ex["scales"]])
        np.testing.assert_allclose(st.scales[h], ex_s, rtol=4e-6, atol=0)
        for r in range(dv):
            for c in range(dk):
                got, want = int(st.codes[h, r, c]), ex["codes"][r][c]
                if got == want:
                    continue
                y, yp = ex["y"][r][c], ex["yp"][r][c]
                band = BAND * (1 + abs(float(y)) + abs(float(yp)))
                assert abs(got - want) == 1 and _boundary_distance(y, yp, rnd) <= band, \
                    (h, r, c, got, want, float(y), float(yp))
                excused += 1
    assert excused <= 2
