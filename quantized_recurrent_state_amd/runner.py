"""Workload set-up around the C ABI: handles, fp32 warmup, calibration, inputs.

Step t of a workload uses the inputs drawn for step index t; a persistent
workload first runs W unquantised (fp32) steps from S_0 = 0 (step indices
0..W-1), freezes the group scales of S_W (lsq_state_calibrate) and then runs
its quantised steps from index W.  This is the persistent-scale set-up of the
workloads: scales frozen from the group absmax of the fp32 state after 64
unquantised warmup steps; every other workload starts quantised from S_0 = 0.
"""
from __future__ import annotations

import torch

from . import LsqConfig, LsqState, POLICY_NONE, POLICY_PERSISTENT, ROUND_RNE
from .inputs import Arm, Workload, gen_steps


def arm_config(wl: Workload, arm: Arm, heads_per_layer: int | None = None) -> LsqConfig:
    d = wl.arm_config(arm)
    if heads_per_layer is not None:          # reduced copy for tests
        d["batch"], d["heads"] = heads_per_layer * len(arm.layers), 1
    return LsqConfig(**d)


def fp32_config(cfg: LsqConfig) -> LsqConfig:
    return LsqConfig(cfg.batch, cfg.heads, cfg.dk, cfg.dv, 32, 1, POLICY_NONE, ROUND_RNE,
                     cfg.delta, cfg.decay)


def inputs(wl: Workload, arm: Arm, t0: int, steps: int, n_per_layer: int, device) -> dict:
    """Inputs of steps [t0, t0+steps) for this arm's layers (seed = layer index)."""
    return gen_steps(wl.recipe, n_per_layer, wl.dk, wl.dv, arm.layers, t0, steps, device=device)


def prepare(wl: Workload, arm: Arm, device, n_per_layer: int | None = None, chunk: int = 8,
            keep_fp32: bool = False):
    """Create the arm's handle at S_0 = 0 and, for a persistent arm, run the fp32
    warmup and calibrate.  Returns (state, first quantised step index, S_W or None)."""
    npl = n_per_layer if n_per_layer is not None else wl.batch * wl.heads
    cfg = arm_config(wl, arm, None if n_per_layer is None else npl)
    st = LsqState(cfg, device=device).zero()
    if arm.policy != POLICY_PERSISTENT or wl.warmup == 0:
        return st, 0, None
    f = LsqState(fp32_config(cfg), device=device).zero()
    for t0 in range(0, wl.warmup, chunk):
        n = min(chunk, wl.warmup - t0)
        d = inputs(wl, arm, t0, n, npl, device)
        f.run(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        del d
    st.calibrate(f.f32)
    S_W = f.f32 if keep_fp32 else None
    del f
    return st, wl.warmup, S_W


def algorithmic_bytes(cfg: LsqConfig, with_o_ref: bool = False) -> int:
    """Bytes one decode step must move for this handle (all heads): packed codes
    read and written, group scales read (and written by the dynamic and yoked
    policies), the yoked fp32 reference read and written, the step inputs
    q, k, v, alpha, beta read and the output o (and o_ref) written."""
    from . import POLICY_DYNAMIC, POLICY_YOKED, DECAY_DIAG
    n, dk, dv = cfg.n, cfg.dk, cfg.dv
    if cfg.bits == 32:
        state = 2 * 4 * dv * dk
    else:
        state = 2 * dv * dk * cfg.bits // 8
        sbytes = 4 if cfg.scale_fmt == 0 else 2
        nscale = dv * (dk // cfg.group) if cfg.group else 1     # group 0: one scale per head
        state += nscale * sbytes * (2 if cfg.policy in (POLICY_DYNAMIC, POLICY_YOKED) else 1)
        if cfg.policy == POLICY_YOKED:
            state += 2 * 4 * dv * dk
    ins = 4 * (2 * dk + dv + (dk if cfg.decay == DECAY_DIAG else 1) + 1)
    outs = 4 * dv * (2 if (with_o_ref and cfg.policy == POLICY_YOKED) else 1)
    lrb = 0
    if cfg.lrb_rank > 0:
        # bypass slots, averaged over a merge period: step j of the period reads
        # the j filled slots (a [Dv], b [Dk]) and, unless it merges, writes the
        # new slot and the slots its decay changed (a under scalar decay, b
        # under diagonal decay)
        r, diag = cfg.lrb_rank, cfg.decay == DECAY_DIAG
        tot = 0
        for j in range(r):
            tot += j * (dv + dk)
            if j < r - 1:
                tot += (dv + dk) + j * (dk if diag else dv)
        lrb = 4 * tot // r
    return n * (state + ins + outs + lrb)


def state_kib_per_head(cfg: LsqConfig) -> int:
    """Packed state of one head (codes and group scales) in KiB, rounded to a
    span the streaming probe supports (1, 2, 4, 8, 10 or 16)."""
    per = cfg.dv * cfg.dk * cfg.bits // 8
    if cfg.bits != 32:
        per += cfg.dv * (cfg.dk // cfg.group if cfg.group else 0) * (4 if cfg.scale_fmt == 0 else 2)
    kib = per / 1024
    return min((1, 2, 4, 8, 10, 16), key=lambda s: abs(s - kib))


def prefill_algorithmic_bytes(cfg: LsqConfig, T: int) -> int:
    """Bytes one prefill of T tokens must move for this handle (all heads): the
    inputs k, v, alpha, beta read once, the packed codes read and written, the
    group scales read (and written by the dynamic policy)."""
    from . import POLICY_DYNAMIC, DECAY_DIAG
    n, dk, dv = cfg.n, cfg.dk, cfg.dv
    ins = 4 * T * (dk + dv + (dk if cfg.decay == DECAY_DIAG else 1) + 1)
    state = 2 * dv * dk * cfg.bits // 8
    state += dv * (dk // cfg.group) * 4 * (2 if cfg.policy == POLICY_DYNAMIC else 1)
    return n * (ins + state)


def prefill_int8_ops(cfg: LsqConfig, T: int) -> int:
    """Integer operations of the chunk products H = V^T K over T tokens (2 per MAC)."""
    return 2 * cfg.n * T * cfg.dk * cfg.dv
