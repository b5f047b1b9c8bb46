"""Exact-rational reference for pinning the oracle (test helper).

Everything here is computed in fractions.Fraction from the fp32 input values,
in the matrix form of Eq. (1) (LinQuant summary, Theoretical Foundation):

    S_t = S_{t-1} Lambda_t (I - delta beta_t k_t k_t^T) + beta_t v_t k_t^T

and the codes are chosen by exhaustive search over the integer grid:
nearest code, ties to even, then clamp ('When Dynamic Scaling Fails': group-wise
symmetric quantisation with a scale per group), and for Bounded Directional
Rounding ('Preserving Updates...', abstract) the nearest code among those that
do not move opposite to the element's update.  Nothing here calls or mirrors
the oracle's row-by-row code path.
"""
from __future__ import annotations

from fractions import Fraction as Fr
import math

POLICY_DYNAMIC, POLICY_PERSISTENT, POLICY_YOKED = 1, 2, 3


def fr(x) -> Fr:
    return Fr(float(x))


def matmul(A, B):
    return [[sum((A[i][l] * B[l][j] for l in range(len(B))), Fr(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def eq1(S_prev, q, k, v, alpha, beta, delta, diag):
    """One exact step of Eq. (1) in matrix form; returns (S_t, o_t, w, S')
    with w the per-row write coefficient and S' = S_{t-1} Lambda_t."""
    dv, dk = len(S_prev), len(S_prev[0])
    K = [[fr(x)] for x in k]                      # column vector
    Kt = [[fr(x) for x in k]]                     # row vector
    V = [[fr(x)] for x in v]
    b = fr(beta)
    Lam = [[(fr(alpha[i]) if diag else fr(alpha)) if i == j else Fr(0) for j in range(dk)]
           for i in range(dk)]
    I = [[Fr(int(i == j)) for j in range(dk)] for i in range(dk)]
    KKt = matmul(K, Kt)
    M = [[I[i][j] - delta * b * KKt[i][j] for j in range(dk)] for i in range(dk)]
    Sp = matmul(S_prev, Lam)
    VKt = matmul(V, Kt)
    S = matmul(Sp, M)
    S = [[S[i][j] + b * VKt[i][j] for j in range(dk)] for i in range(dv)]
    o = [sum((S[i][j] * fr(q[j]) for j in range(dk)), Fr(0)) for i in range(dv)]
    u = [sum((Sp[i][j] * K[j][0] for j in range(dk)), Fr(0)) for i in range(dv)]
    w = [b * (fr(v[i]) - delta * u[i]) for i in range(dv)]
    return S, o, w, Sp


def nearest_even(y: Fr, allowed=lambda c: True) -> int:
    """Nearest integer to y among the allowed ones (searched exhaustively around
    y), ties to even."""
    lo = math.floor(y) - 3
    best = None
    for c in range(lo, lo + 8):
        if not allowed(c):
            continue
        d = abs(Fr(c) - y)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    if best is None:   # every candidate excluded: the constraint lies beyond the window
        raise ValueError("no allowed code near y")
    return best[1]


def bdr_allowed_nearest(y: Fr, yp: Fr, sigma: int) -> int:
    """Nearest integer to y among c with (c - y') * sigma >= 0, ties to even."""
    if sigma == 0:
        return nearest_even(y)
    if sigma > 0:
        lo = math.ceil(yp)
        if lo > math.floor(y) + 1:        # only codes far above y qualify: the smallest
            return lo
        return nearest_even(y, lambda c: c >= yp)
    hi = math.floor(yp)
    if hi < math.ceil(y) - 1:
        return hi
    return nearest_even(y, lambda c: c <= yp)


def sign(x) -> int:
    return (x > 0) - (x < 0)


def quantised_step_exact(cfg: dict, codes_prev, scales_prev, ref_prev, q, k, v, alpha, beta):
    """Exact reference of one quantised step for one head.

    Returns dict with codes, scales (exact Fractions), o, and per element the
    exact code-unit values y (updated) and yp (pre-update) used for the
    boundary band."""
    dv, dk, g = cfg["dv"], cfg["dk"], cfg["group"]
    qmax = (1 << (cfg["bits"] - 1)) - 1
    diag = cfg["decay"] == 1
    S_prev = [[Fr(int(codes_prev[r][c])) * fr(scales_prev[r][c // g]) for c in range(dk)]
              for r in range(dv)]
    S, o, w, Sp = eq1(S_prev, q, k, v, alpha, beta, cfg["delta"], diag)
    R = None
    if cfg["policy"] == POLICY_YOKED:
        R_prev = [[fr(x) for x in row] for row in ref_prev]
        R, _, _, _ = eq1(R_prev, q, k, v, alpha, beta, cfg["delta"], diag)
    codes = [[0] * dk for _ in range(dv)]
    scales = [[Fr(0)] * (dk // g) for _ in range(dv)]
    ys = [[Fr(0)] * dk for _ in range(dv)]
    yps = [[Fr(0)] * dk for _ in range(dv)]
    for r in range(dv):
        for gi in range(dk // g):
            cols = range(gi * g, (gi + 1) * g)
            if cfg["policy"] == POLICY_PERSISTENT:
                s = fr(scales_prev[r][gi])
            else:
                src = R if cfg["policy"] == POLICY_YOKED else S
                s = max(abs(src[r][c]) for c in cols) / qmax
            scales[r][gi] = s
            for c in cols:
                if s == 0:
                    continue
                y = S[r][c] / s
                yp = Sp[r][c] / s
                ys[r][c], yps[r][c] = y, yp
                if cfg["rounding"] == 1:
                    cc = bdr_allowed_nearest(y, yp, sign(w[r]) * sign(fr(k[c])))
                else:
                    cc = nearest_even(y)
                codes[r][c] = max(-qmax, min(qmax, cc))
    return {"codes": codes, "scales": scales, "o": o, "S": S, "R": R, "y": ys, "yp": yps}


def fr_to_f32(x: Fr) -> "np.float32":
    """Round an exact rational to the nearest fp32, ties to even (no double rounding)."""
    import numpy as np
    f = np.float32(float(x))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fr(float(cand)) - x)
        even = (int(np.array(cand).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, cand)
    return np.float32(best[1])
