"""Teacher-forced parity between the HIP path and the CPU oracle (test helper).

A quantised trajectory cannot be compared free-running: one legitimate +-1
code at a rounding boundary changes every later step.  So each step is checked
teacher-forced: the oracle starts from the GPU's own state before the step
(codes, scales, reference), takes the same inputs, and its result is compared
with the GPU's state after the step.

Bar (taken from the decode-step contract):
  * codes bit-exact, except a code that differs by exactly 1 where the
    oracle's exact pre-rounding value lies within BAND_REL * qmax code units of
    the decision boundary (the half-integer of round-half-even, or for
    directional rounding the pre-update value y' against the candidate code,
    for dithered rounding the integers against y + u); such cases are counted
    and reported;
  * dynamic and yoked scales within 1e-6 relative, persistent scales exact;
    16-bit stored scales (binary16, bfloat16) equal, or under the delta rule
    adjacent values of the format (the fp32 scale before rounding may sit at
    the format's rounding midpoint and then follows the dot product's
    summation order); such a group's codes are not compared and the group is
    counted (excused_groups);
  * outputs o (and o_ref) with ||o_gpu - o_oracle||_inf <= 1e-4 ||o_oracle||_inf
    per head;
  * the yoked fp32 reference state within 1e-5 of its own row norm.
The only arithmetic the two sides may do differently is the summation order of
the two row dot products; everything else is specified operation by operation.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle
from oracle import (OracleConfig, OracleState, POLICY_YOKED, POLICY_PERSISTENT, ROUND_BDR,
                    ROUND_DITHER)

BAND_REL = 1e-6
O_TOL = 1e-4
REF_TOL = 1e-5
SCALE_TOL = 1e-6


def ocfg_of(cfg, step: int = 0) -> OracleConfig:
    """The oracle configuration of a GPU handle's configuration; `step` is the
    handle's step index before the step (the dither's sequence position)."""
    return OracleConfig(batch=cfg.batch, heads=cfg.heads, dk=cfg.dk, dv=cfg.dv, bits=cfg.bits,
                        group=cfg.group, policy=cfg.policy, rounding=cfg.rounding,
                        delta=cfg.delta, decay=cfg.decay, step=step,
                        scale_fmt=cfg.scale_fmt)


def snapshot(gpu_state, heads=None) -> OracleState:
    """Device state -> unpacked host state (optionally a subset of heads)."""
    cfg = gpu_state.cfg
    sel = (lambda t: t) if heads is None else (lambda t: t[heads])
    st = OracleState()
    if gpu_state.codes is not None:
        st.codes = oracle.unpack(sel(gpu_state.codes).cpu().numpy(), cfg.bits, cfg.dk)
        st.scales = sel(gpu_state.scales).float().cpu().numpy().copy()
    if gpu_state.ref is not None:
        st.ref = sel(gpu_state.ref).cpu().numpy().copy()
    if gpu_state.f32 is not None:
        st.f32 = sel(gpu_state.f32).cpu().numpy().copy()
    return st


@dataclass
class Report:
    codes: int = 0
    exact: int = 0
    excused: int = 0
    failed: int = 0
    max_o_rel: float = 0.0
    max_oref_rel: float = 0.0
    max_scale_rel: float = 0.0
    max_ref_rel: float = 0.0
    bdr_fired: int = 0
    clamped: int = 0
    excused_groups: int = 0
    groups: int = 0
    notes: list = field(default_factory=list)

    def add(self, o: "Report"):
        for k in ("codes", "exact", "excused", "failed", "bdr_fired", "clamped", "excused_groups",
                  "groups"):
            setattr(self, k, getattr(self, k) + getattr(o, k))
        for k in ("max_o_rel", "max_oref_rel", "max_scale_rel", "max_ref_rel"):
            setattr(self, k, max(getattr(self, k), getattr(o, k)))
        self.notes += o.notes

    @property
    def ok(self) -> bool:
        return (self.failed == 0 and self.max_o_rel <= O_TOL and self.max_oref_rel <= O_TOL
                and self.max_scale_rel <= SCALE_TOL and self.max_ref_rel <= REF_TOL)

    def __str__(self):
        return (f"codes={self.codes} exact={self.exact} excused={self.excused} "
                f"failed={self.failed} o_rel={self.max_o_rel:.2e} oref_rel={self.max_oref_rel:.2e} "
                f"scale_rel={self.max_scale_rel:.2e} ref_rel={self.max_ref_rel:.2e} "
                f"bdr={self.bdr_fired} clamped={self.clamped} "
                f"excused_groups={self.excused_groups}/{self.groups} {self.notes[:3]}")


def _normwise(got, want):
    """max over heads of ||got - want||_inf / ||want||_inf (0/0 -> 0)."""
    got = np.asarray(got, np.float64).reshape(got.shape[0], -1)
    want = np.asarray(want, np.float64).reshape(want.shape[0], -1)
    num = np.abs(got - want).max(axis=1)
    den = np.abs(want).max(axis=1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), np.where(num > 0, np.inf, 0))
    return float(rel.max()) if rel.size else 0.0


def _bits16(scales, fmt):
    """16-bit patterns of scales held as fp32 values of a 16-bit format."""
    x = np.ascontiguousarray(scales, np.float32)
    if fmt == 1:
        return x.astype(np.float16).view(np.uint16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def boundary_distance(y, yp, codes_oracle, rounding):
    """Distance of the exact values to the decision boundary of each element."""
    if rounding == ROUND_DITHER:
        # floor(y + u): the boundaries are the integers (yp holds the dither u)
        z = y + yp
        return np.abs(z - np.round(z))
    d = np.abs(y - (np.floor(y) + 0.5))
    d = np.minimum(d, np.abs(y - (np.floor(y) - 0.5)))
    d = np.minimum(d, np.abs(y - (np.floor(y) + 1.5)))
    if rounding == ROUND_BDR:
        # the reversal test compares a candidate code with y'
        d = np.minimum(d, np.abs(yp - np.round(yp)))
    return d


def compare_step(ocfg: OracleConfig, before: OracleState, inputs, gpu_after: OracleState,
                 gpu_o, gpu_o_ref=None, oracle_after: list | None = None) -> Report:
    """Run the oracle from the GPU's pre-step state and compare with the GPU's result
    (the oracle's post-step state is appended to ``oracle_after`` when given)."""
    rep = Report()
    st = before.copy()
    trace, stats = {}, {}
    o, o_ref = oracle.step(ocfg, st, *inputs, stats=stats, trace=trace)
    if oracle_after is not None:
        oracle_after.append(st)
    rep.max_o_rel = _normwise(np.asarray(gpu_o), o)
    if ocfg.bits == 32:
        rep.max_ref_rel = _normwise(gpu_after.f32, st.f32)
        return rep
    rep.bdr_fired, rep.clamped = stats["bdr_fired"], stats["clamped"]
    if ocfg.policy == POLICY_YOKED:
        rep.max_ref_rel = _normwise(gpu_after.ref, st.ref)
        if gpu_o_ref is not None:
            rep.max_oref_rel = _normwise(np.asarray(gpu_o_ref), o_ref)
    # scales
    skip = np.zeros(st.codes.shape, bool)      # elements of excused groups
    rep.groups = st.scales.size
    if getattr(ocfg, "scale_fmt", 0) and ocfg.policy != POLICY_PERSISTENT:
        g16 = _bits16(gpu_after.scales, ocfg.scale_fmt)
        w16 = _bits16(st.scales, ocfg.scale_fmt)
        diff = g16 != w16
        adjacent = np.abs(g16.astype(np.int64) - w16.astype(np.int64)) == 1
        if np.any(diff & ~adjacent) or (np.any(diff) and ocfg.delta == 0):
            rep.max_scale_rel = np.inf
            rep.notes.append(f"16-bit scales differ at {np.argwhere(diff)[:3].tolist()}")
        rep.excused_groups = int(diff.sum())
        skip = np.repeat(diff, ocfg.group, axis=-1)
    elif ocfg.policy == POLICY_PERSISTENT:
        if not np.array_equal(gpu_after.scales, st.scales):
            rep.max_scale_rel = np.inf
            rep.notes.append("persistent scales changed")
    else:
        den = np.abs(st.scales.astype(np.float64))
        num = np.abs(gpu_after.scales.astype(np.float64) - st.scales)
        rel = np.where(den > 0, num / np.where(den > 0, den, 1), np.where(num > 0, np.inf, 0))
        rep.max_scale_rel = float(rel.max()) if rel.size else 0.0
    # codes
    rep.codes = st.codes.size - int(skip.sum())
    diff = (gpu_after.codes != st.codes) & ~skip
    nd = int(diff.sum())
    rep.exact = rep.codes - nd
    if nd:
        dc = np.abs(gpu_after.codes.astype(np.int32) - st.codes.astype(np.int32))[diff]
        dist = boundary_distance(trace["y"][diff], trace["yp"][diff], st.codes[diff],
                                 ocfg.rounding)
        band = BAND_REL * ocfg.qmax
        ok = (dc == 1) & (dist <= band)
        rep.excused = int(ok.sum())
        rep.failed = int((~ok).sum())
        if rep.failed:
            idx = np.argwhere(diff)[~ok][:3]
            rep.notes.append(f"first failing elements (head,row,col): {idx.tolist()}, "
                             f"dist={dist[~ok][:3].tolist()}, dcode={dc[~ok][:3].tolist()}")
    return rep
