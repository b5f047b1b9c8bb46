"""Pins of the oracle's 16-bit group-scale formats (binary16, bfloat16).

A scale is rounded to its stored format as soon as it is computed, and the
codes are formed with the stored value.  Tied here to:
  * the format conversions of independent libraries: numpy's float32 ->
    float16 cast (round to nearest even, subnormals, overflow to infinity) and
    torch's float32 -> bfloat16 cast, on random values over a wide range, on
    exact ties and at the range ends;
  * the special case where every scale is representable: the 16-bit formats
    then reproduce the fp32-scale oracle bit for bit;
  * a group constructed so that one element's code differs between the
    stored scale and the unrounded one (codes use the stored scale);
  * the quantiser bound with a rounded scale: every element within half a
    stored step, or clamped at qmax with the error the scale's rounding allows.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import OracleConfig, SCALE_BF16, SCALE_F16, SCALE_F32


def _probe_values():
    rng = np.random.default_rng(5)
    wide = np.exp2(rng.uniform(-30, 17, 4000)).astype(np.float32)
    # exact binary16 ties: a representable half value plus half its quantum
    h = rng.integers(1024, 2048, 300).astype(np.float64) * np.exp2(rng.integers(-24, 5, 300))
    q = np.exp2(np.floor(np.log2(h)) - 10)
    ties16 = (h + q / 2).astype(np.float32)
    # bfloat16 ties: 16 discarded bits equal to 0x8000
    b = (rng.integers(0x3000, 0x4700, 300).astype(np.uint32) << 16) | 0x8000
    tiesbf = b.view(np.float32)
    ends = np.array([0.0, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -14, 65504.0, 65519.99,
                     65520.0, 1e6, 3.4e38, 1e-40], np.float32)
    sub = (rng.integers(1, 1024, 200) * 2.0 ** -24 + 2.0 ** -26).astype(np.float32)
    return np.concatenate([wide, ties16, tiesbf, ends, sub])


def test_binary16_rounding_matches_numpy():
    x = _probe_values()
    got = np.array([oracle.scale_as_stored(v, SCALE_F16) for v in x], np.float32)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float32)
    assert np.array_equal(got, want, equal_nan=True)


def test_bfloat16_rounding_matches_torch():
    x = _probe_values()
    got = np.array([oracle.scale_as_stored(v, SCALE_BF16) for v in x], np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, want)


def test_fp32_format_is_the_identity():
    x = _probe_values()
    assert np.array_equal(np.array([oracle.scale_as_stored(v, SCALE_F32) for v in x], np.float32), x)


def _cfg(fmt, policy=oracle.POLICY_DYNAMIC, rounding=oracle.ROUND_RNE, bits=4, delta=1, decay=0):
    return OracleConfig(batch=1, heads=2, dk=64, dv=8, bits=bits, group=32, policy=policy,
                        rounding=rounding, delta=delta, decay=decay, scale_fmt=fmt)


@pytest.mark.parametrize("fmt", [SCALE_F16, SCALE_BF16])
@pytest.mark.parametrize("policy,rounding", [(oracle.POLICY_DYNAMIC, oracle.ROUND_RNE),
                                             (oracle.POLICY_PERSISTENT, oracle.ROUND_BDR),
                                             (oracle.POLICY_YOKED, oracle.ROUND_RNE)])
def test_representable_scales_reproduce_the_fp32_oracle(fmt, policy, rounding):
    """States whose group maxima are qmax times a power of two have scales
    exact in every format: the result equals the fp32-scale oracle's."""
    rng = np.random.default_rng(11)
    bits = 4
    qm = 7
    S = rng.uniform(-1, 1, (2, 8, 64)).astype(np.float32)
    g = S.reshape(2, 8, 2, 32)
    top = np.exp2(rng.integers(-6, 3, (2, 8, 2))).astype(np.float32) * qm
    g /= np.abs(g).max(-1, keepdims=True)
    g *= top[..., None]
    S = g.reshape(2, 8, 64).astype(np.float32)
    c16, c32 = _cfg(fmt, policy, rounding, bits, delta=0), _cfg(SCALE_F32, policy, rounding, bits, delta=0)
    a, b = oracle.calibrate(c16, S), oracle.calibrate(c32, S)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
    if policy == oracle.POLICY_PERSISTENT:
        # one step with k = 0: the state only decays by 1/2 (exact); the frozen
        # scales are representable, so the step matches too
        z = np.zeros((2, 64), np.float32)
        v = np.zeros((2, 8), np.float32)
        oracle.step(c16, a, z, z, v, np.full(2, 0.5, np.float32), np.ones(2, np.float32))
        oracle.step(c32, b, z, z, v, np.full(2, 0.5, np.float32), np.ones(2, np.float32))
        assert np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)


def test_codes_are_formed_with_the_stored_scale():
    """A group whose fp32 scale s is just above its binary16 value h: an
    element at 2.5 h (1 + 2^-20) lies above the tie on h's grid (code 3) but
    below it on s's grid (code 2)."""
    h = np.float32(2.0 ** -4 * (1 + 5 * 2.0 ** -10))          # a binary16 value
    s_target = np.float32(h * np.float32(1 + 2.0 ** -13))      # rounds to h in binary16
    assert np.float32(s_target).astype(np.float16).astype(np.float32) == h
    amax = np.float32(7 * s_target)
    assert np.float32(amax / np.float32(7)) != h               # the fp32 scale differs from h
    x = np.float32(2.5 * h * (1 + 2.0 ** -20))
    row = np.zeros(32, np.float32)
    row[0] = amax
    row[1] = x
    S = np.zeros((2, 8, 64), np.float32)
    S[0, 0, :32] = row
    st = oracle.calibrate(_cfg(SCALE_F16, bits=4, delta=0), S)
    assert st.scales[0, 0, 0] == h
    assert st.codes[0, 0, 1] == 3
    assert st.codes[0, 0, 0] == 7                              # amax / h > 7: clamped
    st32 = oracle.calibrate(_cfg(SCALE_F32, bits=4, delta=0), S)
    assert st32.codes[0, 0, 1] == 2


@pytest.mark.parametrize("fmt", [SCALE_F16, SCALE_BF16])
@pytest.mark.parametrize("bits", [4, 8])
def test_rounded_scales_keep_the_quantiser_bound(fmt, bits):
    rng = np.random.default_rng(2)
    cfg = _cfg(fmt, bits=bits, delta=0)
    qm = cfg.qmax
    S = (rng.standard_normal((2, 8, 64)) * np.exp2(rng.integers(-8, 4, (2, 8, 1)))).astype(np.float32)
    st = oracle.calibrate(cfg, S)
    s = st.scales
    rep = np.array([oracle.scale_as_stored(v, fmt) for v in s.ravel()], np.float32).reshape(s.shape)
    assert np.array_equal(rep, s)                              # stored values are in the format
    deq = oracle.dequantize(cfg, st).astype(np.float64)
    se = np.repeat(s, 32, axis=-1).astype(np.float64)
    exact = np.repeat(np.abs(S).reshape(2, 8, 2, 32).max(-1) / qm, 32, axis=-1)
    err = np.abs(deq - S)
    clamped = np.abs(st.codes) == qm
    assert np.all(err[~clamped] <= 0.5 * se[~clamped] * (1 + 1e-6))
    # a clamped element exceeds qmax steps only by the scale's rounding
    assert np.all(err[clamped] <= 0.5 * se[clamped] + qm * np.abs(exact - se)[clamped] * (1 + 1e-6))
