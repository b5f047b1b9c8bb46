"""Pins of the oracle's recurrence against closed forms of Eq. (1).

Eq. (1) of the LinQuant summary (Theoretical Foundation):
    S_t = S_{t-1} Lambda_t (I - delta beta_t k_t k_t^T) + beta_t v_t k_t^T,
with scalar decay Lambda_t = alpha_t I or diagonal decay diag(alpha_t)
(Key structural choices).  With delta = 0 the state is a decayed sum of the
written associations; with delta = 1, beta = 1 and orthonormal keys, reading
the state with key k_j returns v_j (scaled by the later decays).
"""
import numpy as np
import pytest

import oracle
from oracle import OracleConfig, POLICY_NONE, DECAY_SCALAR, DECAY_DIAG

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _fp32_cfg(n, dk, dv, delta, decay):
    return OracleConfig(batch=n, heads=1, dk=dk, dv=dv, bits=32, group=1, policy=POLICY_NONE,
                        delta=delta, decay=decay)


def _rand(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _run_fp32(cfg, T, q, k, v, a, b):
    st = oracle.zero_state(cfg)
    o, _ = oracle.run(cfg, st, q, k, v, a, b)
    return st.f32.astype(np.float64), o


@pytest.mark.parametrize("dk,dv", [(8, 8), (16, 5), (4, 12)])
def test_linear_write_is_sum_of_outer_products(dk, dv):
    """delta = 0, alpha = 1: S_T = sum_t beta_t v_t k_t^T."""
    rng = np.random.default_rng(1)
    n, T = 3, 40
    cfg = _fp32_cfg(n, dk, dv, 0, DECAY_SCALAR)
    q, k, v = _rand(rng, (T, n, dk)), _rand(rng, (T, n, dk)), _rand(rng, (T, n, dv))
    a = np.ones((T, n), np.float32)
    b = rng.uniform(0.1, 1.0, (T, n)).astype(np.float32)
    S, _ = _run_fp32(cfg, T, q, k, v, a, b)
    ref = np.einsum("tn,tnr,tnc->nrc", b.astype(np.float64), v.astype(np.float64),
                    k.astype(np.float64))
    np.testing.assert_allclose(S, ref, rtol=0, atol=2e-5 * np.abs(ref).max())


def test_scalar_decay_closed_form():
    """S_T = sum_t (prod_{tau>t} alpha_tau) beta_t v_t k_t^T."""
    rng = np.random.default_rng(2)
    n, dk, dv, T = 4, 8, 6, 30
    cfg = _fp32_cfg(n, dk, dv, 0, DECAY_SCALAR)
    q, k, v = _rand(rng, (T, n, dk)), _rand(rng, (T, n, dk)), _rand(rng, (T, n, dv))
    a = rng.uniform(0.7, 1.0, (T, n)).astype(np.float32)
    b = rng.uniform(0.1, 1.0, (T, n)).astype(np.float32)
    S, _ = _run_fp32(cfg, T, q, k, v, a, b)
    a64 = a.astype(np.float64)
    ref = np.zeros((n, dv, dk))
    for t in range(T):
        later = np.prod(a64[t + 1:], axis=0)           # [n]
        ref += (later * b[t])[:, None, None] * np.einsum("nr,nc->nrc", v[t], k[t])
    np.testing.assert_allclose(S, ref, rtol=0, atol=2e-5 * np.abs(ref).max())


def test_diagonal_decay_acts_on_key_columns():
    """Lambda_t = diag(alpha_t) multiplies S from the right: column c decays by alpha_{t,c}."""
    rng = np.random.default_rng(3)
    n, dk, dv, T = 2, 8, 5, 25
    cfg = _fp32_cfg(n, dk, dv, 0, DECAY_DIAG)
    q, k, v = _rand(rng, (T, n, dk)), _rand(rng, (T, n, dk)), _rand(rng, (T, n, dv))
    a = rng.uniform(0.5, 1.0, (T, n, dk)).astype(np.float32)
    b = rng.uniform(0.1, 1.0, (T, n)).astype(np.float32)
    S, _ = _run_fp32(cfg, T, q, k, v, a, b)
    a64 = a.astype(np.float64)
    ref = np.zeros((n, dv, dk))
    for t in range(T):
        later = np.prod(a64[t + 1:], axis=0)           # [n, dk]
        ref += b[t][:, None, None] * np.einsum("nr,nc->nrc", v[t], k[t] * later)
    np.testing.assert_allclose(S, ref, rtol=0, atol=2e-5 * np.abs(ref).max())


@pytest.mark.parametrize("decayed", [False, True])
def test_delta_rule_recalls_with_orthonormal_keys(decayed):
    """delta = 1, beta = 1, orthonormal keys: S_n k_j = (prod_{i>j} alpha_i) v_j."""
    rng = np.random.default_rng(4)
    dk, dv, nk = 16, 7, 12
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :nk].T.astype(np.float32)          # nk orthonormal rows
    cfg = _fp32_cfg(1, dk, dv, 1, DECAY_SCALAR)
    k = keys[:, None, :]
    v = _rand(rng, (nk, 1, dv))
    q = np.zeros((nk, 1, dk), np.float32)
    a = (rng.uniform(0.8, 1.0, (nk, 1)) if decayed else np.ones((nk, 1))).astype(np.float32)
    b = np.ones((nk, 1), np.float32)
    S, _ = _run_fp32(cfg, nk, q, k, v, a, b)
    for j in range(nk):
        scale = np.prod(a[j + 1:, 0].astype(np.float64))
        np.testing.assert_allclose(S[0] @ keys[j].astype(np.float64), scale * v[j, 0],
                                   rtol=0, atol=2e-6 * (1 + np.abs(v).max()))


def test_delta_rule_one_hot_keys_overwrite():
    """With one-hot keys the delta rule overwrites column j with v_j (up to the one
    fp32 rounding of v - S'k and of the write) and leaves every other column
    bit-identical."""
    rng = np.random.default_rng(5)
    dk, dv = 6, 4
    cfg = _fp32_cfg(1, dk, dv, 1, DECAY_SCALAR)
    order = [2, 0, 5, 2, 3]                           # key 2 is written twice
    T = len(order)
    k = np.zeros((T, 1, dk), np.float32)
    for t, j in enumerate(order):
        k[t, 0, j] = 1.0
    v = _rand(rng, (T, 1, dv))
    st = oracle.zero_state(cfg)
    # warm the state with a dense write first so the overwrite is visible
    w0 = _rand(rng, (1, 1, dk))
    oracle.run(cfg, st, np.zeros((1, 1, dk), np.float32), w0, _rand(rng, (1, 1, dv)),
               np.ones((1, 1), np.float32), np.ones((1, 1), np.float32))
    before = st.f32.copy()
    oracle.run(cfg, st, np.zeros((T, 1, dk), np.float32), k, v, np.ones((T, 1), np.float32),
               np.ones((T, 1), np.float32))
    last = {j: t for t, j in enumerate(order)}
    for c in range(dk):
        if c in last:
            got, want = st.f32[0, :, c], v[last[c], 0]
            assert np.all(np.abs(got - want) <= 2.0 ** -22 * (np.abs(want) + np.abs(before).max()))
        else:
            assert np.array_equal(st.f32[0, :, c], before[0, :, c])


@pytest.mark.parametrize("delta,decay", [(0, DECAY_SCALAR), (1, DECAY_SCALAR), (0, DECAY_DIAG),
                                         (1, DECAY_DIAG)])
def test_matches_matrix_form_of_eq1(delta, decay):
    """General inputs: the oracle's row form follows the matrix recursion of Eq. (1)
    (Dv != Dk, so a transposed operand cannot pass)."""
    rng = np.random.default_rng(6 + delta + 2 * decay)
    n, dk, dv, T = 2, 12, 5, 20
    cfg = _fp32_cfg(n, dk, dv, delta, decay)
    q = _rand(rng, (T, n, dk))
    k = _rand(rng, (T, n, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = _rand(rng, (T, n, dv))
    a = rng.uniform(0.6, 1.0, (T, n, dk) if decay == DECAY_DIAG else (T, n)).astype(np.float32)
    b = rng.uniform(0.1, 1.0, (T, n)).astype(np.float32)
    S, o = _run_fp32(cfg, T, q, k, v, a, b)
    ref = np.zeros((n, dv, dk))
    ref_o = np.zeros((T, n, dv))
    I = np.eye(dk)
    for t in range(T):
        for h in range(n):
            Lam = np.diag(a[t, h]) if decay == DECAY_DIAG else a[t, h] * I
            kk = k[t, h].astype(np.float64)
            ref[h] = (ref[h] @ Lam @ (I - delta * b[t, h] * np.outer(kk, kk))
                      + b[t, h] * np.outer(v[t, h], kk))
            ref_o[t, h] = ref[h] @ q[t, h]
    np.testing.assert_allclose(S, ref, rtol=0, atol=1e-5 * np.abs(ref).max())
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-5 * np.abs(ref_o).max())


def test_readout_is_state_times_query():
    """o_t = S_t q_t, read from the updated state (a library matvec in fp64)."""
    rng = np.random.default_rng(9)
    n, dk, dv = 3, 10, 7
    cfg = _fp32_cfg(n, dk, dv, 1, DECAY_SCALAR)
    st = oracle.zero_state(cfg)
    for _ in range(5):
        q, k, v = _rand(rng, (n, dk)), _rand(rng, (n, dk)), _rand(rng, (n, dv))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        o, _ = oracle.step(cfg, st, q, k, v, np.full(n, 0.9, np.float32),
                           np.full(n, 0.5, np.float32))
        ref = np.einsum("nrc,nc->nr", st.f32.astype(np.float64), q.astype(np.float64))
        np.testing.assert_allclose(o, ref, rtol=1e-6, atol=1e-7)
