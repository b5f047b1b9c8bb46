"""Pins of the oracle's Low-Rank Bypass step (lsqo_step_lrb).

"Preserving Updates in Low-Bit Recurrent State Quantization" (abstract) names
the method in one sentence; the oracle's reading (lsq_oracle.h): r fp32
rank-one slots take each step's write, the delta projection and the readout
see S' + B, and every r-th step the buffer is merged into the quantised state.
Tied here to things other than its own code:
  * r = 1 is the plain decode step (every step merges its own write): codes and
    scales equal lsqo_step's bit for bit, o agrees to fp32 accuracy;
  * between merges, with unit decay, the codes do not move, and the readout is
    the dense recursion o_t = (S_0 + sum_{s<=t} w_s k_s^T) q_t with
    w_s = beta (v_s - delta (S_0 + B_{s-1}) k_s), recomputed here in fp64;
  * with decay, the buffer decays like the state: the dense recursion with
    B <- B Lambda_t before each write;
  * a merge requantises S' + B: the codes equal the quantiser applied to the
    fp64 dense sum except within 1e-6 of a rounding boundary.
"""
import numpy as np
import pytest

import oracle
from oracle import OracleConfig


def _inputs(rng, n, dk, dv):
    q = rng.standard_normal((n, dk)).astype(np.float32)
    k = rng.standard_normal((n, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv)).astype(np.float32)
    return q, k, v


@pytest.mark.parametrize("rnd", [oracle.ROUND_RNE, oracle.ROUND_BDR, oracle.ROUND_DITHER])
@pytest.mark.parametrize("pol", [oracle.POLICY_DYNAMIC, oracle.POLICY_PERSISTENT])
@pytest.mark.parametrize("decay", [oracle.DECAY_SCALAR, oracle.DECAY_DIAG])
def test_rank_one_bypass_is_the_plain_step(rnd, pol, decay):
    rng = np.random.default_rng(5)
    n, dk, dv = 3, 64, 8
    base = OracleConfig(batch=1, heads=n, dk=dk, dv=dv, bits=4, group=32, policy=pol,
                        rounding=rnd, delta=1, decay=decay)
    S0 = (rng.standard_normal((n, dv, dk)) * 0.2).astype(np.float32)
    plain = oracle.calibrate(base, S0)
    lrb = oracle.calibrate(base.replace(lrb_rank=1), S0)
    lrb.lrb_a = np.zeros((n, 1, dv), np.float32)
    lrb.lrb_b = np.zeros((n, 1, dk), np.float32)
    for t in range(6):
        q, k, v = _inputs(rng, n, dk, dv)
        a = (rng.uniform(0.8, 1.0, (n, dk)) if decay else rng.uniform(0.8, 1.0, n)).astype(np.float32)
        b = rng.uniform(0.2, 1.0, n).astype(np.float32)
        o1, _ = oracle.step(base.replace(step=t), plain, q, k, v, a, b)
        o2, _ = oracle.step(base.replace(lrb_rank=1, step=t), lrb, q, k, v, a, b)
        assert np.array_equal(plain.codes, lrb.codes), t
        assert np.array_equal(plain.scales, lrb.scales), t
        assert np.abs(o1 - o2).max() <= 1e-5 * max(1.0, np.abs(o1).max())


def _dense_recursion(S0_deq, steps, delta, R, decays):
    """fp64 effective state S_0 + B over the steps before the first merge."""
    B = np.zeros_like(S0_deq, dtype=np.float64)
    S = S0_deq.astype(np.float64)
    outs = []
    for (q, k, v, a, b), lam in zip(steps, decays):
        S = S * lam
        B = B * lam
        X = S + B
        u = np.einsum("nij,nj->ni", X, k) if delta else 0.0
        w = b[:, None] * (v - u)
        B = B + w[:, :, None] * k[:, None, :]
        outs.append(np.einsum("nij,nj->ni", S + B, q))
    return outs, S + B


@pytest.mark.parametrize("delta", [0, 1])
@pytest.mark.parametrize("decay", [oracle.DECAY_SCALAR, oracle.DECAY_DIAG])
def test_between_merges_the_readout_follows_the_dense_recursion(delta, decay):
    rng = np.random.default_rng(11)
    n, dk, dv, R = 2, 64, 16, 6
    cfg = OracleConfig(batch=1, heads=n, dk=dk, dv=dv, bits=8, group=64,
                       policy=oracle.POLICY_PERSISTENT, rounding=oracle.ROUND_RNE, delta=delta,
                       decay=decay, lrb_rank=R)
    S0 = (rng.standard_normal((n, dv, dk)) * 0.3).astype(np.float32)
    st = oracle.calibrate(cfg, S0)
    st.lrb_a = np.zeros((n, R, dv), np.float32)
    st.lrb_b = np.zeros((n, R, dk), np.float32)
    deq = oracle.dequantize(cfg, st)
    codes0 = st.codes.copy()
    steps, lams, outs = [], [], []
    for t in range(R - 1):                    # no merge yet
        q, k, v = _inputs(rng, n, dk, dv)
        if decay:
            a = np.ones((n, dk), np.float32)  # unit decay keeps the codes fixed
            lam = np.ones((n, 1, dk))
        else:
            a = np.ones(n, np.float32)
            lam = np.ones((n, 1, 1))
        b = rng.uniform(0.2, 1.0, n).astype(np.float32)
        o, _ = oracle.step(cfg.replace(step=t), st, q, k, v, a, b)
        steps.append((q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), a, b))
        lams.append(lam)
        outs.append(o)
        assert np.array_equal(st.codes, codes0)
    want, _ = _dense_recursion(deq, steps, delta, R, lams)
    for o, w in zip(outs, want):
        assert np.abs(o - w).max() <= 1e-5 * np.abs(w).max()


@pytest.mark.parametrize("decay", [oracle.DECAY_SCALAR, oracle.DECAY_DIAG])
def test_buffer_decays_like_the_state_and_merge_requantises_the_sum(decay):
    rng = np.random.default_rng(21)
    n, dk, dv, R = 2, 64, 16, 4
    cfg = OracleConfig(batch=1, heads=n, dk=dk, dv=dv, bits=8, group=32,
                       policy=oracle.POLICY_DYNAMIC, rounding=oracle.ROUND_RNE, delta=1,
                       decay=decay, lrb_rank=R)
    st = oracle.zero_state(cfg)                 # S_0 = 0: S' stays 0 until the merge
    steps, lams, outs = [], [], []
    for t in range(R):
        q, k, v = _inputs(rng, n, dk, dv)
        if decay:
            a = rng.uniform(0.7, 1.0, (n, dk)).astype(np.float32)
            lam = a[:, None, :].astype(np.float64)
        else:
            a = rng.uniform(0.7, 1.0, n).astype(np.float32)
            lam = a[:, None, None].astype(np.float64)
        b = rng.uniform(0.2, 1.0, n).astype(np.float32)
        tr = {}
        o, _ = oracle.step(cfg.replace(step=t), st, q, k, v, a, b, trace=tr)
        steps.append((q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), a, b))
        lams.append(lam)
        outs.append(o)
        if t < R - 1:
            assert not st.codes.any()             # nothing merged yet
    want, X = _dense_recursion(np.zeros((n, dv, dk)), steps, 1, R, lams)
    for o, w in zip(outs, want):
        assert np.abs(o - w).max() <= 1e-5 * np.abs(w).max()
    # the merge: dynamic absmax scales and RNE codes of the dense sum
    g = cfg.group
    Xg = X.reshape(n, dv, dk // g, g)
    s = np.abs(Xg).max(axis=-1) / 127.0
    assert np.allclose(st.scales, s, rtol=1e-5)
    y = X / np.repeat(st.scales.astype(np.float64), g, axis=-1)
    near = np.abs(np.abs(y - np.floor(y)) - 0.5) < 1e-4
    ref = np.clip(np.round(y), -127, 127)
    assert np.array_equal(st.codes[~near], ref[~near].astype(np.int8))
    assert near.sum() < 5


def test_merge_period_and_slot_reuse():
    """Codes change exactly on steps r-1, 2r-1, ...; the second period starts empty."""
    rng = np.random.default_rng(2)
    n, dk, dv, R = 1, 64, 8, 3
    cfg = OracleConfig(batch=1, heads=n, dk=dk, dv=dv, bits=4, group=64,
                       policy=oracle.POLICY_PERSISTENT, rounding=oracle.ROUND_RNE, delta=0,
                       lrb_rank=R)
    st = oracle.zero_state(cfg)
    st.scales[:] = 0.05
    changed = []
    prev = st.codes.copy()
    for t in range(3 * R):
        q, k, v = _inputs(rng, n, dk, dv)
        oracle.step(cfg.replace(step=t), st, q, k, v, np.ones(n, np.float32),
                    np.ones(n, np.float32))
        changed.append(not np.array_equal(prev, st.codes))
        prev = st.codes.copy()
    assert changed == [(t % R) == R - 1 for t in range(3 * R)]
