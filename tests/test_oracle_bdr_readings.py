"""Pins of the two directional-rounding readings that were not taken (A, B'),
kept behind rounding flags for sensitivity runs (persistent scale only).

  A   the update is the total change from the stored value C_old s:
      sigma = sign(S_t - C_old s); a reversal is c1 on the far side of C_old;
  B'  the update is the rank-one write, sigma = sign(w) sign(k_c), and the move
      is measured from the stored value: reversal as in A.

Tied here to:
  * a theorem: on a frozen grid RNE is monotone, so reading A never finds a
    reversal and equals round-to-nearest-even bit for bit (random inputs,
    every decay and delta mode, many steps);
  * a hand-worked step (one row, frozen scale 1, decay 1/2) where the decay
    carries an element below its stored code and the write cannot bring it
    back: B' returns the stored code, the taken reading and RNE do not;
  * B' properties: at most one step from RNE, only where the write has a
    direction and RNE landed on the far side of the stored code (the fix stays
    between c1 and C_old, so the clamp after it never acts);
  * both flags are refused with a scale that is not frozen.
"""
import numpy as np
import pytest

import oracle
from oracle import OracleConfig, ROUND_BDR, ROUND_BDR_A, ROUND_BDR_B, ROUND_RNE


def _cfg(rounding, bits=4, dk=64, dv=16, delta=0, decay=0, n=3, group=32):
    return OracleConfig(batch=1, heads=n, dk=dk, dv=dv, bits=bits, group=group,
                        policy=oracle.POLICY_PERSISTENT, rounding=rounding, delta=delta,
                        decay=decay)


def _inputs(rng, cfg):
    n, dk, dv = cfg.n, cfg.dk, cfg.dv
    k = rng.standard_normal((n, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((n, dk)).astype(np.float32)
    v = rng.standard_normal((n, dv)).astype(np.float32)
    a = (rng.uniform(0.9, 1.0, (n, dk)) if cfg.decay else rng.uniform(0.9, 1.0, n)).astype(np.float32)
    b = rng.uniform(0.2, 1.0, n).astype(np.float32)
    return q, k, v, a, b


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("delta,decay", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_reading_A_equals_rne_on_a_frozen_grid(bits, delta, decay):
    rng = np.random.default_rng(bits * 10 + delta * 2 + decay)
    ca, cr = _cfg(ROUND_BDR_A, bits, delta=delta, decay=decay), _cfg(ROUND_RNE, bits, delta=delta, decay=decay)
    S0 = (rng.standard_normal((ca.n, ca.dv, ca.dk)) * 0.5).astype(np.float32)
    sa, sr = oracle.calibrate(ca, S0), oracle.calibrate(cr, S0)
    fired = 0
    for t in range(40):
        x = _inputs(rng, ca)
        stats = {}
        oa, _ = oracle.step(ca, sa, *x, stats=stats)
        orr, _ = oracle.step(cr, sr, *x)
        fired += stats["bdr_fired"]
        assert np.array_equal(sa.codes, sr.codes) and np.array_equal(oa, orr), t
    assert fired == 0


def _worked(rounding):
    """One row of 32 elements, INT4, frozen scale 1, scalar decay 1/2, beta 1,
    v = 0.3, no delta rule.  Elements: 0: C_old 3, k 1; 1: C_old -2, k 1;
    2: C_old 3, k -1; 3: C_old 3, k 0; the rest 0 with k 0."""
    cfg = OracleConfig(batch=1, heads=1, dk=32, dv=1, bits=4, group=32,
                       policy=oracle.POLICY_PERSISTENT, rounding=rounding)
    st = oracle.zero_state(cfg)
    st.codes[0, 0, :4] = [3, -2, 3, 3]
    st.scales[:] = 1.0
    k = np.zeros((1, 32), np.float32)
    k[0, :3] = [1.0, 1.0, -1.0]
    z = np.zeros((1, 32), np.float32)
    oracle.step(cfg, st, z, k, np.full((1, 1), 0.3, np.float32), np.full(1, 0.5, np.float32),
                np.ones(1, np.float32))
    return st.codes[0, 0, :4].tolist()


def test_worked_step_separates_the_readings():
    # S' = C_old / 2 = [1.5, -1, 1.5, 1.5]; S = S' + 0.3 k = [1.8, -0.7, 1.2, 1.5]
    assert _worked(ROUND_RNE) == [2, -1, 1, 2]        # RNE (1.5 ties to 2)
    assert _worked(ROUND_BDR) == [2, -1, 1, 2]        # from S': no reversal
    assert _worked(ROUND_BDR_A) == [2, -1, 1, 2]      # total change: all moved down or up consistently
    # B': element 0 has an upward write but RNE (2) lies below the stored 3:
    # one step toward the write; element 2's write points down, 1 < 3 agrees
    assert _worked(ROUND_BDR_B) == [3, -1, 1, 2]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("delta,decay", [(0, 0), (1, 1)])
def test_reading_B_moves_at_most_one_step_toward_the_write(bits, delta, decay):
    rng = np.random.default_rng(7 + bits + delta)
    cb, cr = _cfg(ROUND_BDR_B, bits, delta=delta, decay=decay), _cfg(ROUND_RNE, bits, delta=delta, decay=decay)
    S0 = (rng.standard_normal((cb.n, cb.dv, cb.dk)) * 0.5).astype(np.float32)
    st = oracle.calibrate(cb, S0)
    fired = 0
    qm = cb.qmax
    for t in range(20):
        q, k, v, a, b = _inputs(rng, cb)
        before = st.copy()
        # the RNE result and the write's sign from the same pre-step state
        ref = before.copy()
        trace = {}
        oracle.step(cr, ref, q, k, v, a, b)
        stats = {}
        oracle.step(cb, st, q, k, v, a, b, stats=stats, trace=trace)
        fired += stats["bdr_fired"]
        c1, c2, cold = ref.codes.astype(int), st.codes.astype(int), before.codes.astype(int)
        d = c2 - c1
        assert np.all(np.abs(d) <= 1)
        moved = d != 0
        # where it moved, RNE had landed on the far side of the stored code and
        # the fix points from c1 back toward it, within the clamp
        assert np.all(((c1 - cold) * d)[moved] < 0)
        assert np.all(np.abs(c2) <= qm)
        assert int(moved.sum()) == stats["bdr_fired"]
    assert fired > 0


@pytest.mark.parametrize("rounding", [ROUND_BDR_A, ROUND_BDR_B])
@pytest.mark.parametrize("policy", [oracle.POLICY_DYNAMIC, oracle.POLICY_YOKED])
def test_flags_need_a_frozen_scale(rounding, policy):
    cfg = _cfg(rounding).replace(policy=policy)
    with pytest.raises(Exception):
        oracle.step(cfg, oracle.zero_state(cfg), *_inputs(np.random.default_rng(0), cfg))
