"""Pins of the oracle's chunkwise prefill state pass (lsqo_prefill).

The LinQuant summary (Methodology, Low-Precision Chunkwise Realization) writes
the chunk state as H = Q(B V)^T Q(Gamma-> (.) K) and passes it on with
S_[i+1] = Q(gamma^C S_[i] + H).  Tied here to things other than its own code:
  * operands chosen on the INT8 grids: one chunk reproduces the exact sum of
    v_t k_t^T to within half a state step per element;
  * the chunk recursion against the token-by-token fp32 recurrence of Eq. (1)
    (the oracle's unquantised mode, delta = 0), within the error the operand
    and state quantisers allow, for scalar and diagonal decay, with a short
    last chunk;
  * the decay bookkeeping in closed form: a lone token t of a chunk enters H
    with the product of the later decays, a^(C-1-t) for a constant a, and a
    chunk without writes multiplies the state by the product of all its decays;
  * the recursion's Q(.) at every chunk boundary: writes below half a state
    step vanish across chunks but add up inside one;
  * INT8 operand codes round half to even (exact ties exposed through the
    dynamic state scale);
  * a binary16 stored scale forms the codes (numpy's rounding of the exact
    group absmax over qmax);
  * one scale per head: the dynamic scale covers all of the head's X, and a
    frozen head scale is the same quantiser as group scales sharing it;
  * T = 0 changes nothing.
"""
import numpy as np
import pytest

import oracle
from oracle import OracleConfig


def _cfg(n=2, dk=64, dv=32, bits=8, group=32, policy=oracle.POLICY_DYNAMIC, decay=0):
    return OracleConfig(batch=1, heads=n, dk=dk, dv=dv, bits=bits, group=group, policy=policy,
                        rounding=oracle.ROUND_RNE, delta=0, decay=decay)


def test_grid_operands_give_the_exact_sum_within_half_a_step():
    rng = np.random.default_rng(1)
    cfg = _cfg()
    T = 40                                   # one chunk
    v = rng.integers(-127, 128, (T, 2, 32)) * 2.0 ** -7
    k = rng.integers(-127, 128, (T, 2, 64)) * 2.0 ** -10
    v[0, :, 0] = 127 * 2.0 ** -7             # absmax on the grid: scale 2^-7 exactly
    k[0, :, 0] = 127 * 2.0 ** -10
    st = oracle.zero_state(cfg)
    oracle.prefill(cfg, st, k, v, np.ones((T, 2)), np.ones((T, 2)), chunk=64)
    X = np.einsum("tni,tnj->nij", v, k)      # exact in float64
    deq = oracle.dequantize(cfg, st)
    s = np.repeat(st.scales, 32, axis=-1)
    assert np.all(np.abs(deq - X) <= 0.5 * s * (1 + 1e-6))
    Xg = np.abs(X).reshape(2, 32, 2, 32).max(-1)
    assert np.allclose(st.scales, Xg / 127, rtol=1e-6)


def test_a_binary16_dynamic_scale_forms_the_codes():
    """A stored binary16 scale (the scale-format reading): with grid operands one
    chunk from a zero state makes X exact, so the stored scale must be numpy's
    binary16 rounding of fl(max|X| / qmax) and every code the round-half-even
    of X times the fp32 reciprocal of that stored value, clamped."""
    rng = np.random.default_rng(2)
    cfg = _cfg().replace(scale_fmt=oracle.SCALE_F16)
    T = 40
    v = rng.integers(-127, 128, (T, 2, 32)) * 2.0 ** -7
    k = rng.integers(-127, 128, (T, 2, 64)) * 2.0 ** -10
    v[0, :, 0] = 127 * 2.0 ** -7
    k[0, :, 0] = 127 * 2.0 ** -10
    st = oracle.zero_state(cfg)
    oracle.prefill(cfg, st, k, v, np.ones((T, 2)), np.ones((T, 2)), chunk=64)
    X = np.einsum("tni,tnj->nij", v, k)                         # exact, and fp32-representable
    amax = np.abs(X).reshape(2, 32, 2, 32).max(-1).astype(np.float32)
    s16 = (amax / np.float32(127)).astype(np.float16).astype(np.float32)
    assert np.array_equal(st.scales, s16)
    inv = np.where(s16 > 0, np.float32(1) / np.where(s16 > 0, s16, 1), 0).astype(np.float32)
    want = np.clip(np.rint(X * np.repeat(inv, 32, axis=-1).astype(np.float64)), -127, 127)
    assert np.array_equal(st.codes, want.astype(np.int8))
    # and the stored value differs from the fp32 scale somewhere, so the pin bites
    assert np.any(s16 != amax / np.float32(127))


def test_a_dynamic_head_scale_covers_the_whole_head():
    """One scale per head (group 0): with grid operands one chunk from a zero
    state makes X exact, so the head's scale must be fl(max over all of its
    X / qmax) and every code the round-half-even of X times its reciprocal."""
    rng = np.random.default_rng(4)
    cfg = _cfg(group=0)
    T = 40
    v = rng.integers(-127, 128, (T, 2, 32)) * 2.0 ** -7
    k = rng.integers(-127, 128, (T, 2, 64)) * 2.0 ** -10
    v[0, :, 0] = 127 * 2.0 ** -7
    k[0, :, 0] = 127 * 2.0 ** -10
    st = oracle.zero_state(cfg)
    oracle.prefill(cfg, st, k, v, np.ones((T, 2)), np.ones((T, 2)), chunk=64)
    X = np.einsum("tni,tnj->nij", v, k)
    s = (np.abs(X).reshape(2, -1).max(-1).astype(np.float32) / np.float32(127)).astype(np.float32)
    assert np.array_equal(st.scales.reshape(2), s)
    inv = (np.float32(1) / s).astype(np.float64)
    want = np.clip(np.rint(X * inv[:, None, None]), -127, 127)
    assert np.array_equal(st.codes, want.astype(np.int8))


@pytest.mark.parametrize("decay", [0, 1])
def test_a_frozen_head_scale_equals_groups_sharing_it(decay):
    """A persistent scale per head s is the same quantiser as group scales all
    equal to s: the two prefills agree bit for bit over several chunks."""
    rng = np.random.default_rng(5)
    T = 150
    k = rng.standard_normal((T, 2, 64)).astype(np.float32) / 8
    v = rng.standard_normal((T, 2, 32)).astype(np.float32)
    a = (rng.uniform(0.9, 1.0, (T, 2, 64)) if decay else rng.uniform(0.9, 1.0, (T, 2))).astype(np.float32)
    b = rng.uniform(0.2, 1.0, (T, 2)).astype(np.float32)
    C0 = rng.integers(-127, 128, (2, 32, 64)).astype(np.int8)
    s_head = np.array([0.011, 0.027], np.float32)
    ch = _cfg(group=0, policy=oracle.POLICY_PERSISTENT, decay=decay)
    cg = _cfg(group=32, policy=oracle.POLICY_PERSISTENT, decay=decay)
    sh, sg = oracle.zero_state(ch), oracle.zero_state(cg)
    sh.codes[:] = C0
    sg.codes[:] = C0
    sh.scales[:] = s_head.reshape(sh.scales.shape)
    sg.scales[:] = s_head[:, None, None]
    oracle.prefill(ch, sh, k, v, a, b, chunk=64)
    oracle.prefill(cg, sg, k, v, a, b, chunk=64)
    assert np.array_equal(sh.codes, sg.codes)
    assert np.any(sh.codes != C0)


@pytest.mark.parametrize("decay", [0, 1])
@pytest.mark.parametrize("T", [64, 100, 192])
def test_chunks_follow_the_token_recurrence(decay, T):
    rng = np.random.default_rng(7)
    n, dk, dv = 2, 64, 32
    cfg = _cfg(n=n, dk=dk, dv=dv, decay=decay)
    k = rng.standard_normal((T, n, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, dv)).astype(np.float32)
    if decay:
        a = rng.uniform(0.95, 1.0, (T, n, dk)).astype(np.float32)
    else:
        a = rng.uniform(0.95, 1.0, (T, n)).astype(np.float32)
    b = rng.uniform(0.3, 1.0, (T, n)).astype(np.float32)
    st = oracle.zero_state(cfg)
    oracle.prefill(cfg, st, k, v, a, b, chunk=64)
    # the unquantised token recurrence (q is irrelevant for the state)
    fcfg = cfg.replace(bits=32, policy=oracle.POLICY_NONE)
    fst = oracle.zero_state(fcfg)
    oracle.run(fcfg, fst, np.zeros_like(k), k, v, a, b)
    deq = oracle.dequantize(cfg, st)
    ref = fst.f32
    err = np.abs(deq - ref).max() / np.abs(ref).max()
    assert err < 0.03, err                   # INT8 operands and state: a few 1/127 steps


def test_a_lone_token_enters_with_the_product_of_later_decays():
    n, dk, dv, C = 1, 64, 32, 16
    cfg = _cfg(n=n, dk=dk, dv=dv, policy=oracle.POLICY_PERSISTENT)
    a = 0.8
    k1 = np.zeros(dk, np.float32); k1[3] = 1.0
    v1 = np.zeros(dv, np.float32); v1[5] = 1.0
    vals = []
    for t in range(C):
        k = np.zeros((C, n, dk), np.float32); k[t, 0] = k1
        v = np.zeros((C, n, dv), np.float32); v[t, 0] = v1
        st = oracle.zero_state(cfg)
        st.scales[:] = 2.0 ** -6                # state step 1/64, range +-1.98
        oracle.prefill(cfg, st, k, v, np.full((C, n), a, np.float32), np.ones((C, n), np.float32),
                       chunk=C)
        vals.append(float(oracle.dequantize(cfg, st)[0, 5, 3]))
    # the operand quantiser maps a lone token's block to 127 exactly: H = a^(C-1-t)
    want = [a ** (C - 1 - t) for t in range(C)]
    assert np.allclose(vals, want, rtol=0, atol=2.0 ** -7)   # half a state step


def test_a_chunk_without_writes_decays_the_state():
    rng = np.random.default_rng(3)
    n, dk, dv, C = 2, 64, 16, 32
    cfg = _cfg(n=n, dk=dk, dv=dv, policy=oracle.POLICY_PERSISTENT, group=64)
    S = rng.standard_normal((n, dv, dk)).astype(np.float32)
    st = oracle.calibrate(cfg, S)
    c0 = st.codes.astype(np.float64)
    a = rng.uniform(0.9, 1.0, (C, n)).astype(np.float32)
    z = np.zeros((C, n, dk), np.float32)
    oracle.prefill(cfg, st, z, np.zeros((C, n, dv), np.float32), a, np.ones((C, n), np.float32),
                   chunk=C)
    gam = np.ones(n, np.float32)
    for t in range(C - 1, -1, -1):           # the chunk's product of decays, in fp32
        gam = (gam * a[t]).astype(np.float32)
    want = np.clip(np.round(c0 * gam[:, None, None].astype(np.float64)), -127, 127)
    near = np.abs(np.abs(c0 * gam[:, None, None] - np.floor(c0 * gam[:, None, None])) - 0.5) < 1e-5
    assert np.array_equal(st.codes[~near], want[~near])


def test_empty_prompt_changes_nothing():
    cfg = _cfg()
    st = oracle.calibrate(cfg, np.random.default_rng(0).standard_normal((2, 32, 64)).astype(np.float32))
    before = st.copy()
    oracle.prefill(cfg, st, np.zeros((0, 2, 64)), np.zeros((0, 2, 32)), np.zeros((0, 2)),
                   np.zeros((0, 2)))
    assert np.array_equal(st.codes, before.codes) and np.array_equal(st.scales, before.scales)


def test_the_state_is_requantised_at_every_chunk_boundary():
    """S_[i+1] = Q(gamma^C S_[i] + H): a write worth 0.49 of a state step is
    rounded away at the end of its chunk, so two such writes in consecutive
    chunks leave the state at 0, while the same two writes inside one chunk
    add exactly (integer product) to 0.98 and round to 1."""
    n, dk, dv, C = 1, 32, 16, 64
    cfg = _cfg(n=n, dk=dk, dv=dv, policy=oracle.POLICY_PERSISTENT)

    def prefill(tokens):
        T = 2 * C
        k = np.zeros((T, n, dk), np.float32)
        v = np.zeros((T, n, dv), np.float32)
        for t in tokens:
            v[t, 0, 0] = 127 * 2.0 ** -7     # s_V = 2^-7, code 127
            k[t, 0, 0] = 127 * 2.0 ** -8     # s_K = 2^-8, code 127
        st = oracle.zero_state(cfg)
        st.scales[:] = 1.0                   # H = 127^2 2^-15 = 0.4922 state steps per write
        oracle.prefill(cfg, st, k, v, np.ones((T, n), np.float32), np.ones((T, n), np.float32),
                       chunk=C)
        return st.codes
    assert not prefill([0, C]).any()
    once = prefill([0, 1])
    assert once[0, 0, 0] == 1 and np.count_nonzero(once) == 1


def test_operand_codes_round_half_to_even():
    """INT8 operand codes at exact ties: 2.5 -> 2 and 3.5 -> 4.  One token with
    k = 127 2^-7 e_0 gives H[r][0] = c_r 127 2^-14, so the dynamic scale of row r
    is c_r 2^-14 exactly and exposes the operand code c_r."""
    n, dk, dv = 1, 32, 16
    cfg = _cfg(n=n, dk=dk, dv=dv, group=32)
    k = np.zeros((1, n, dk), np.float32)
    v = np.zeros((1, n, dv), np.float32)
    k[0, 0, 0] = 127 * 2.0 ** -7
    v[0, 0, :3] = np.array([127, 2.5, 3.5]) * 2.0 ** -7
    st = oracle.zero_state(cfg)
    oracle.prefill(cfg, st, k, v, np.ones((1, n), np.float32), np.ones((1, n), np.float32))
    assert st.scales[0, 0, 0] == 127 * 2.0 ** -14
    assert st.scales[0, 1, 0] == 2 * 2.0 ** -14
    assert st.scales[0, 2, 0] == 4 * 2.0 ** -14
    assert np.all(st.codes[0, :3, 0] == 127)
