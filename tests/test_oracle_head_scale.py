"""Pins of the oracle's per-head scale (group = 0: one scale for the whole
Dv x Dk state of a head, the coarsest of the scale granularities).

Tied here to:
  * the group path it must reduce to: with one row per head (Dv = 1) a
    per-head scale is a per-row scale, so the per-head step equals the pinned
    group = Dk step bit for bit (dynamic and persistent, RNE and BDR, both
    decays, with and without the delta rule, several steps), and calibration
    likewise;
  * quantiser invariants of the whole-head dynamic scale: no element clamps,
    some element of every non-zero head reaches qmax, rows of small magnitude
    keep codes well below qmax (the scale is not taken per row), and every
    element is within half a step of S_t;
  * a frozen per-head scale never changes.
"""
import numpy as np
import pytest

import oracle
from oracle import OracleConfig


def _cfg(group, dv, policy, rounding, delta, decay, bits=4, n=3, dk=64):
    return OracleConfig(batch=1, heads=n, dk=dk, dv=dv, bits=bits, group=group, policy=policy,
                        rounding=rounding, delta=delta, decay=decay)


def _inputs(rng, n, dk, dv, decay, vscale=None):
    k = rng.standard_normal((n, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((n, dk)).astype(np.float32)
    v = rng.standard_normal((n, dv)).astype(np.float32)
    if vscale is not None:
        v = (v * vscale).astype(np.float32)
    a = (rng.uniform(0.9, 1.0, (n, dk)) if decay else rng.uniform(0.9, 1.0, n)).astype(np.float32)
    b = rng.uniform(0.2, 1.0, n).astype(np.float32)
    return q, k, v, a, b


@pytest.mark.parametrize("policy", [oracle.POLICY_DYNAMIC, oracle.POLICY_PERSISTENT])
@pytest.mark.parametrize("rounding", [oracle.ROUND_RNE, oracle.ROUND_BDR])
@pytest.mark.parametrize("delta,decay", [(0, 0), (1, 1)])
@pytest.mark.parametrize("bits", [4, 8])
def test_one_row_heads_equal_the_row_group_path(policy, rounding, delta, decay, bits):
    rng = np.random.default_rng(bits + 3 * delta + 5 * rounding + 7 * policy)
    dk = 64
    ch = _cfg(0, 1, policy, rounding, delta, decay, bits)
    cg = _cfg(dk, 1, policy, rounding, delta, decay, bits)
    S0 = (rng.standard_normal((3, 1, dk)) * 0.4).astype(np.float32)
    sh, sg = oracle.calibrate(ch, S0), oracle.calibrate(cg, S0)
    assert np.array_equal(sh.codes, sg.codes)
    assert np.array_equal(sh.scales.ravel(), sg.scales.ravel())
    for t in range(12):
        x = _inputs(rng, 3, dk, 1, decay)
        oh, _ = oracle.step(ch, sh, *x)
        og, _ = oracle.step(cg, sg, *x)
        assert np.array_equal(sh.codes, sg.codes), t
        assert np.array_equal(sh.scales.ravel(), sg.scales.ravel()), t
        assert np.array_equal(oh, og), t


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("rounding", [oracle.ROUND_RNE, oracle.ROUND_BDR])
def test_dynamic_head_scale_spans_all_rows(bits, rounding):
    rng = np.random.default_rng(20 + bits)
    n, dk, dv = 3, 64, 24
    cfg = _cfg(0, dv, oracle.POLICY_DYNAMIC, rounding, 1, 0, bits, n=n, dk=dk)
    st = oracle.zero_state(cfg)
    vscale = np.where(np.arange(dv) < dv // 2, 1.0, 0.05)     # half the rows 20x smaller
    for t in range(10):
        stats, trace = {}, {}
        oracle.step(cfg, st, *_inputs(rng, n, dk, dv, 0, vscale), stats=stats, trace=trace)
        assert stats["clamped"] == 0
        c = np.abs(st.codes.astype(int))
        assert np.all(c.reshape(n, -1).max(-1) == cfg.qmax)
        assert c[:, dv // 2:].max() < cfg.qmax // 4              # small rows: small codes
        # within half a step of S_t = y / inv (rounding only, no clamp)
        y = trace["y"]
        if rounding == oracle.ROUND_RNE:
            assert np.all(np.abs(st.codes - y) <= 0.5)
        else:
            assert np.all(np.abs(st.codes - y) < 1.0)


def test_frozen_head_scale_stays():
    rng = np.random.default_rng(9)
    n, dk, dv = 2, 64, 16
    cfg = _cfg(0, dv, oracle.POLICY_PERSISTENT, oracle.ROUND_BDR, 1, 1, 4, n=n, dk=dk)
    st = oracle.calibrate(cfg, (rng.standard_normal((n, dv, dk)) * 0.3).astype(np.float32))
    s0 = st.scales.copy()
    assert s0.shape == (n, 1, 1)
    for t in range(5):
        oracle.step(cfg, st, *_inputs(rng, n, dk, dv, 1))
    assert np.array_equal(st.scales, s0)
    deq = oracle.dequantize(cfg, st)
    assert np.allclose(deq, st.codes * s0, rtol=0, atol=0)


@pytest.mark.parametrize("change", [dict(policy=oracle.POLICY_YOKED), dict(rounding=oracle.ROUND_DITHER),
                                    dict(lrb_rank=2)])
def test_head_scale_refuses_other_modes(change):
    cfg = _cfg(0, 8, oracle.POLICY_DYNAMIC, oracle.ROUND_RNE, 0, 0).replace(**change)
    with pytest.raises(Exception):
        oracle.step(cfg, oracle.zero_state(cfg), *_inputs(np.random.default_rng(0), 3, 64, 8, 0))


@pytest.mark.parametrize("rounding", [oracle.ROUND_RNE, oracle.ROUND_BDR])
@pytest.mark.parametrize("delta,decay", [(0, 0), (1, 1), (1, 0)])
def test_frozen_head_scale_equals_rows_sharing_that_scale(rounding, delta, decay):
    """A frozen per-head scale acts on each element exactly as a frozen row
    scale of the same value: many-row heads against the group path."""
    rng = np.random.default_rng(31 + delta + rounding)
    n, dk, dv = 2, 64, 12
    ch = _cfg(0, dv, oracle.POLICY_PERSISTENT, rounding, delta, decay, 4, n=n, dk=dk)
    cg = _cfg(32, dv, oracle.POLICY_PERSISTENT, rounding, delta, decay, 4, n=n, dk=dk)
    sh = oracle.calibrate(ch, (rng.standard_normal((n, dv, dk)) * 0.3).astype(np.float32))
    sg = oracle.zero_state(cg)
    sg.codes[:] = sh.codes
    sg.scales[:] = sh.scales.reshape(n, 1, 1)
    for t in range(8):
        x = _inputs(rng, n, dk, dv, decay)
        oh, _ = oracle.step(ch, sh, *x)
        og, _ = oracle.step(cg, sg, *x)
        assert np.array_equal(sh.codes, sg.codes) and np.array_equal(oh, og), t


def test_one_row_heads_with_bfloat16_scales():
    rng = np.random.default_rng(4)
    ch = _cfg(0, 1, oracle.POLICY_DYNAMIC, oracle.ROUND_BDR, 1, 0).replace(scale_fmt=oracle.SCALE_BF16)
    cg = _cfg(64, 1, oracle.POLICY_DYNAMIC, oracle.ROUND_BDR, 1, 0).replace(scale_fmt=oracle.SCALE_BF16)
    sh, sg = oracle.zero_state(ch), oracle.zero_state(cg)
    for t in range(10):
        x = _inputs(rng, 3, 64, 1, 0)
        oracle.step(ch, sh, *x)
        oracle.step(cg, sg, *x)
        assert np.array_equal(sh.codes, sg.codes) and np.array_equal(sh.scales.ravel(), sg.scales.ravel())


@pytest.mark.parametrize("bits", [4, 8])
def test_head_calibration_spans_all_rows(bits):
    rng = np.random.default_rng(40 + bits)
    n, dk, dv = 3, 64, 20
    cfg = _cfg(0, dv, oracle.POLICY_PERSISTENT, oracle.ROUND_RNE, 0, 0, bits, n=n, dk=dk)
    S = (rng.standard_normal((n, dv, dk)) * np.linspace(0.05, 2.0, dv)[None, :, None]).astype(np.float32)
    st = oracle.calibrate(cfg, S)
    s = st.scales.reshape(n, 1, 1).astype(np.float64)
    assert np.all(np.abs(st.codes.astype(int)).reshape(n, -1).max(-1) == cfg.qmax)
    assert np.all(np.abs(st.codes * s - S) <= 0.5 * s * (1 + 1e-6))       # nothing clamped
