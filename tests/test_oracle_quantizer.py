"""Pins of the oracle's quantiser, scale policies and rounding rules.

Sources: 'When Dynamic Scaling Fails' (abstract; project page, mechanism
paragraph): group-wise symmetric INT4/INT8 state requantised every step, the
per-token dynamic scale read from the state being quantised, the persistent
scale, the scale yoked to a full-precision reference.  'Preserving Updates in
Low-Bit Recurrent State Quantization' (abstract): Bounded Directional Rounding
moves reversed elements toward their update, enlarging the rounding error.
"""
import json
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import (OracleConfig, POLICY_DYNAMIC, POLICY_PERSISTENT, POLICY_YOKED, POLICY_NONE,
                    ROUND_RNE, ROUND_BDR, DECAY_SCALAR, DECAY_DIAG)
from tests import exact_ref as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- packed layout
def test_pack_layout_golden():
    d = json.load(open(os.path.join(GOLDEN, "pack_layout.json")))
    for case in d["cases"]:
        codes = np.array([case["codes"]], np.int8)
        packed = oracle.pack(codes, case["bits"])
        assert packed[0].tobytes().hex() == case["bytes_hex"], case["derivation"]
        assert np.array_equal(oracle.unpack(packed, case["bits"], case["dk"]), codes)


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_roundtrip_all_codes(bits):
    qm = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(bits)
    codes = rng.integers(-qm, qm + 1, size=(7, 3, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack(oracle.pack(codes, bits), bits, 64), codes)


# ---------------------------------------------------------------- worked steps
def _golden_state(cfg, case):
    st = oracle.zero_state(cfg)
    st.codes[0] = np.array(case["codes_prev"], np.int8)
    st.scales[0] = np.array(case["scales_prev"], np.float32)
    return st


def _golden_inputs(cfg, case):
    q = np.array([case["q"]], np.float32)
    k = np.array([case["k"]], np.float32)
    v = np.array([case["v"]], np.float32)
    a = np.array([case["alpha"]], np.float32)
    b = np.array([case["beta"]], np.float32)
    return q, k, v, a, b


def test_worked_steps_golden():
    d = json.load(open(os.path.join(GOLDEN, "worked_steps.json")))
    c0, c1 = d["cases"]
    cfg = OracleConfig(**c0["config"])
    st = _golden_state(cfg, c0)
    o, _ = oracle.step(cfg, st, *_golden_inputs(cfg, c0))
    assert o[0].tolist() == c0["expect_o"]
    assert st.codes[0].tolist() == c0["expect_codes"]
    for r, (num, den) in enumerate(c0["expect_scales_exact"]):
        assert st.scales[0, r, 0] == X.fr_to_f32(Fr(num) / Fr(den))   # one rounding of num/den

    for rounding, key in ((ROUND_RNE, "expect_codes_rne"), (ROUND_BDR, "expect_codes_bdr")):
        cfg = OracleConfig(**{**c1["config"], "rounding": rounding})
        st = _golden_state(cfg, c1)
        o, _ = oracle.step(cfg, st, *_golden_inputs(cfg, c1))
        assert o[0].tolist() == c1["expect_o"]
        assert st.codes[0].tolist() == c1[key]
        assert st.scales[0].tolist() == c1["scales_prev"]


# ---------------------------------------------------------------- quantiser invariants
@pytest.mark.parametrize("bits,group", [(4, 32), (8, 64), (4, 8), (8, 16)])
def test_quantise_dequantise_idempotent_on_grid(bits, group):
    """Requantising a dequantised grid state returns the same codes."""
    rng = np.random.default_rng(11 + bits)
    qm = (1 << (bits - 1)) - 1
    n, dv, dk = 3, 4, 64
    cfg = OracleConfig(n, 1, dk, dv, bits, group, POLICY_DYNAMIC, ROUND_RNE)
    codes = rng.integers(-qm, qm + 1, size=(n, dv, dk)).astype(np.int8)
    # each group reaches +-qmax so the absmax scale reproduces the grid
    codes[..., ::group] = qm * rng.choice([-1, 1], size=codes[..., ::group].shape)
    scales = np.exp(rng.uniform(-6, 3, size=(n, dv, dk // group))).astype(np.float32)
    st = oracle.OracleState(codes=codes, scales=scales)
    again = oracle.calibrate(cfg, oracle.dequantize(cfg, st))
    assert np.array_equal(again.codes, codes)
    np.testing.assert_allclose(again.scales, scales, rtol=2 ** -22)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantiser_is_odd(bits):
    rng = np.random.default_rng(21)
    cfg = OracleConfig(2, 1, 64, 8, bits, 32 if bits == 4 else 64, POLICY_DYNAMIC)
    S = rng.standard_normal((2, 8, 64)).astype(np.float32)
    a, b = oracle.calibrate(cfg, S), oracle.calibrate(cfg, -S)
    assert np.array_equal(a.codes, -b.codes)
    assert np.array_equal(a.scales, b.scales)


def test_calibration_reaches_qmax_and_zero_groups_stay_zero():
    rng = np.random.default_rng(22)
    cfg = OracleConfig(2, 1, 128, 16, 4, 32, POLICY_PERSISTENT)
    S = rng.standard_normal((2, 16, 128)).astype(np.float32)
    S[0, 3, 32:64] = 0.0
    st = oracle.calibrate(cfg, S)
    m = np.abs(st.codes.reshape(2, 16, 4, 32)).max(-1)
    assert m[0, 3, 1] == 0 and st.scales[0, 3, 1] == 0.0
    m[0, 3, 1] = 7
    assert np.all(m == 7)


def _gdn_inputs(rng, T, n, dk, dv, diag=False):
    q = rng.standard_normal((T, n, dk)).astype(np.float32)
    k = rng.standard_normal((T, n, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, dv)).astype(np.float32)
    a = rng.uniform(0.9, 1.0, (T, n, dk) if diag else (T, n)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (T, n)).astype(np.float32)
    return q, k, v, a, b


def test_dynamic_scale_each_group_reaches_qmax():
    rng = np.random.default_rng(23)
    cfg = OracleConfig(4, 1, 64, 8, 4, 32, POLICY_DYNAMIC, ROUND_RNE, delta=1)
    st = oracle.zero_state(cfg)
    for t, inp in enumerate(zip(*_gdn_inputs(rng, 12, 4, 64, 8))):
        oracle.step(cfg, st, *inp)
        m = np.abs(st.codes.reshape(4, 8, 2, 32)).max(-1)
        assert np.all((m == 7) | (st.scales == 0))


def test_persistent_scale_is_frozen_and_codes_bounded():
    rng = np.random.default_rng(24)
    cfg = OracleConfig(3, 1, 64, 8, 4, 32, POLICY_PERSISTENT, ROUND_BDR, delta=1)
    st, _ = oracle.fp32_warmup_then_calibrate(cfg, *_gdn_inputs(rng, 16, 3, 64, 8))
    s0 = st.scales.copy()
    stats = {}
    for inp in zip(*_gdn_inputs(rng, 30, 3, 64, 8)):
        oracle.step(cfg, st, *inp, stats=stats)
        assert np.array_equal(st.scales, s0)
        assert np.abs(st.codes).max() <= 7
    assert stats["bdr_fired"] > 0


def test_yoked_reference_is_the_fp32_trajectory():
    """The yoked arm's reference state is exactly an fp32-state run on the same
    inputs (the page's 'full-precision reference running alongside')."""
    rng = np.random.default_rng(25)
    n, dk, dv, T = 3, 64, 8, 20
    cfg = OracleConfig(n, 1, dk, dv, 4, 32, POLICY_YOKED, ROUND_RNE, delta=1)
    fcfg = cfg.replace(bits=32, policy=POLICY_NONE)
    st, fst = oracle.zero_state(cfg), oracle.zero_state(fcfg)
    for inp in zip(*_gdn_inputs(rng, T, n, dk, dv)):
        _, o_ref = oracle.step(cfg, st, *inp)
        o32, _ = oracle.step(fcfg, fst, *inp)
        assert np.array_equal(st.ref, fst.f32)
        assert np.array_equal(o_ref, o32)
        # the scale is read from the reference, not from the quantised state
        want = (np.abs(st.ref.reshape(n, dv, 2, 32)).max(-1) / np.float32(7)).astype(np.float32)
        assert np.array_equal(st.scales, want)


# ---------------------------------------------------------------- BDR properties
def test_bdr_bounded_and_no_reversal_left():
    """After BDR every element is within one grid step of its exact value, and
    no element that could move is left moving opposite to its update."""
    rng = np.random.default_rng(26)
    n, dk, dv = 64, 32, 4
    cfg = OracleConfig(n, 1, dk, dv, 4, 32, POLICY_PERSISTENT, ROUND_BDR, delta=1)
    st, _ = oracle.fp32_warmup_then_calibrate(cfg, *_gdn_inputs(rng, 8, n, dk, dv))
    for inp in zip(*_gdn_inputs(rng, 6, n, dk, dv)):
        prev = st.copy()
        q, k, v, a, b = inp
        oracle.step(cfg, st, *inp)
        # recompute S', w and S in fp32 exactly as written in Eq. (1) row form
        m = prev.scales.repeat(32, -1) * a[:, None, None]
        sp = prev.codes.astype(np.float32) * m
        u = np.einsum("nrc,nc->nr", sp.astype(np.float64), k.astype(np.float64)).astype(np.float32)
        w = b[:, None] * (v - u)
        S = np.array([[[X.fr_to_f32(Fr(float(w[h, r])) * Fr(float(k[h, c])) + Fr(float(sp[h, r, c])))
                        for c in range(dk)] for r in range(dv)] for h in range(n)], np.float32)
        inv = np.where(st.scales == 0, 0, (1 / st.scales.astype(np.float64)).astype(np.float32))
        inv = inv.repeat(32, -1).astype(np.float64)
        y = S.astype(np.float64) * inv
        yp = sp.astype(np.float64) * inv
        c = st.codes.astype(np.float64)
        unclamped = np.abs(c) < 7
        assert np.all(np.abs(c - y)[unclamped] <= 1.0)
        sig = np.sign(w)[..., None] * np.sign(k)[:, None, :]
        reversed_ = ((c - yp) * sig < 0) & unclamped
        assert not reversed_.any()


def test_bdr_enlarges_rounding_error():
    """The abstract: BDR enlarges the rounding error (teacher-forced, same states)."""
    rng = np.random.default_rng(27)
    n, dk, dv = 32, 64, 8
    base = OracleConfig(n, 1, dk, dv, 4, 32, POLICY_PERSISTENT, ROUND_RNE, delta=1)
    st, _ = oracle.fp32_warmup_then_calibrate(base, *_gdn_inputs(rng, 16, n, dk, dv))
    err = {ROUND_RNE: 0.0, ROUND_BDR: 0.0}
    for inp in zip(*_gdn_inputs(rng, 10, n, dk, dv)):
        fp = oracle.OracleState(f32=oracle.dequantize(base, st))
        oracle.step(base.replace(bits=32, policy=POLICY_NONE), fp, *inp)
        for rnd in err:
            s2 = st.copy()
            oracle.step(base.replace(rounding=rnd), s2, *inp)
            err[rnd] += np.abs(oracle.dequantize(base, s2) - fp.f32).mean()
        oracle.step(base, st, *inp)
    assert err[ROUND_BDR] > err[ROUND_RNE]
