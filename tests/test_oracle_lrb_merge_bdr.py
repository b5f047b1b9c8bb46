"""Exact pin of the bypass merge under Bounded Directional Rounding, ranks 2-4.

"Preserving Updates in Low-Bit Recurrent State Quantization" (abstract): small
updates accumulate in a low-rank buffer that is merged into the low-bit state
periodically, and a rounded element that moved opposite to its update is
rounded one grid step toward the update.  The reading (lsq_oracle.h): at the
merge the requantised value is X = S' + sum_j a_j b_j^T, the update whose
direction counts is the buffer's own value U = sum_j a_j b_j^T, and the move
is measured from the decayed pre-merge value S'.

The reference below is independent of the oracle's row code: exact rationals
over a whole merge period, from the inputs (linear write, delta = 0, dyadic
values so that every fp32 operation of the step is exact), with the code chosen
by exhaustive search as "the nearest code to X/s among the codes that do not
move opposite to U from S'/s", ties to even, then clamped.  Two planted
mistakes, the sign of the last write instead of U's and the move measured from
X instead of S', each make the oracle disagree with it.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import OracleConfig
from tests.exact_ref import bdr_allowed_nearest, nearest_even, sign

DK, DV, QMAX = 8, 16, 7


def _draw(rng, r, diag):
    """Dyadic inputs of one merge period: k in quarters (with a zero column),
    v in 32nds up to 1/4 (updates of a fraction of a grid step, where
    reversals happen), beta in {1/2, 1}, decays in {1/2, 3/4, 7/8, 1}."""
    steps = []
    for _ in range(r):
        k = rng.integers(-4, 5, DK).astype(np.float32) / 4
        k[3] = 0.0                                   # a column without update direction
        v = rng.integers(-8, 9, DV).astype(np.float32) / 32
        beta = np.float32(rng.choice([0.5, 1.0]))
        dec = np.array([0.5, 0.75, 0.875, 1.0], np.float32)
        alpha = rng.choice(dec, DK).astype(np.float32) if diag else np.float32(rng.choice(dec))
        steps.append((k, v, alpha, beta))
    return steps


def _period_exact(C0, s, steps, diag):
    """Codes after each step of one period (the last step merges), exact."""
    r = len(steps)
    C = [[int(x) for x in row] for row in C0]
    A, B = [], []                                    # slots: a_j [Dv], b_j [Dk]
    out = []
    for t, (k, v, alpha, beta) in enumerate(steps):
        al = [Fr(float(alpha[c])) if diag else Fr(float(alpha)) for c in range(DK)]
        # the buffer decays with the state
        for j in range(len(A)):
            if diag:
                B[j] = [B[j][c] * al[c] for c in range(DK)]
            else:
                A[j] = [A[j][i] * al[0] for i in range(DV)]
        A.append([Fr(float(beta)) * Fr(float(v[i])) for i in range(DV)])   # w = beta v
        B.append([Fr(float(k[c])) for c in range(DK)])
        merge = t == r - 1
        newC = []
        for i in range(DV):
            si = Fr(float(s[i]))
            row = []
            for c in range(DK):
                sp = C[i][c] * si * al[c]                        # S' = C fl(s alpha), exact here
                if merge:
                    U = sum((A[j][i] * B[j][c] for j in range(r)), Fr(0))
                    y, yp = (sp + U) / si, sp / si
                    code = bdr_allowed_nearest(y, yp, sign(U))
                else:
                    code = nearest_even(sp / si)                 # requantised from S' alone
                row.append(max(-QMAX, min(QMAX, code)))
            newC.append(row)
        C = newC
        out.append(np.array(C, np.int8))
    return out


def _run_oracle(C0, s, steps, diag, r):
    cfg = OracleConfig(batch=1, heads=1, dk=DK, dv=DV, bits=4, group=DK,
                       policy=oracle.POLICY_PERSISTENT, rounding=oracle.ROUND_BDR, delta=0,
                       decay=oracle.DECAY_DIAG if diag else oracle.DECAY_SCALAR, lrb_rank=r)
    st = oracle.zero_state(cfg)
    st.codes[0] = C0
    st.scales[0, :, 0] = s
    q = np.zeros((1, DK), np.float32)
    out, fired = [], 0
    for t, (k, v, alpha, beta) in enumerate(steps):
        a = alpha.reshape(1, DK) if diag else np.array([alpha], np.float32)
        stats = {}
        oracle.step(cfg.replace(step=t), st, q, k.reshape(1, DK), v.reshape(1, DV), a,
                    np.array([beta], np.float32), stats=stats)
        fired += stats["bdr_fired"]
        out.append(st.codes[0].copy())
    return out, fired


CASES = [(r, diag, seed) for r in (2, 3, 4) for diag in (False, True) for seed in range(6)]


def _case(r, diag, seed):
    rng = np.random.default_rng(100 * r + 10 * diag + seed)
    C0 = rng.integers(-QMAX, QMAX + 1, (DV, DK)).astype(np.int8)
    s = np.float32(2.0) ** rng.integers(-4, -1, DV).astype(np.float32)    # 1/16 .. 1/4
    return C0, s, _draw(rng, r, diag)


@pytest.mark.parametrize("r,diag,seed", CASES)
def test_merge_matches_exact_reference(r, diag, seed):
    C0, s, steps = _case(r, diag, seed)
    want = _period_exact(C0, s, steps, diag)
    got, _ = _run_oracle(C0, s, steps, diag, r)
    for t, (g, w) in enumerate(zip(got, want)):
        assert np.array_equal(g, w), (t, np.argwhere(g != w)[:4].tolist())


def test_cases_exercise_the_rule():
    """Across the cases the merge reverses elements, and U's sign differs from
    the last write's where the rounding depends on it (so the pins below bite)."""
    fired = 0
    for r, diag, seed in CASES:
        C0, s, steps = _case(r, diag, seed)
        _, f = _run_oracle(C0, s, steps, diag, r)
        fired += f
    assert fired >= 40


PLANTS = {
    # the direction taken from the last write a_n b_n^T instead of the buffer's value U
    "sign of the last write": [(
        "sig[c] = (uv > 0.0f) - (uv < 0.0f);   /* direction of the accumulated update */",
        "sig[c] = merge ? sign_f(A[n_used * dv + i]) * sign_f(Bv[n_used * dk + c]) : 0;")],
    # the move measured from the merged value X instead of the pre-merge S'
    "move measured from X": [(
        "requantise_group(cfg, i, gi * g, (gi + 1) * g, x, sp, sig, inv, C, &st,",
        "requantise_group(cfg, i, gi * g, (gi + 1) * g, x, x, sig, inv, C, &st,")],
}


@pytest.mark.parametrize("name", sorted(PLANTS))
def test_planted_mistakes_are_caught(name):
    mismatches = 0
    with oracle.planted(PLANTS[name]):
        for r, diag, seed in CASES:
            C0, s, steps = _case(r, diag, seed)
            want = _period_exact(C0, s, steps, diag)
            got, _ = _run_oracle(C0, s, steps, diag, r)
            mismatches += sum(int((g != w).sum()) for g, w in zip(got, want))
    assert mismatches >= 3, (name, mismatches)
