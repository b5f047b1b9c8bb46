"""GPU parity: the HIP decode step against the CPU oracle, element by element.

Every flag combination (bits, Dk, policy, rounding, delta, decay) runs a few
steps on small states whose Dv leaves a ragged tail of rows and whose head
count leaves a partially filled last workgroup; every step is compared
teacher-forced (tests/parity.py states the bar).  The fp32-state mode is
compared free-running over a whole horizon.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_recurrent_state_amd as lsq
from quantized_recurrent_state_amd.inputs import gen_steps
from tests.parity import Report, compare_step, ocfg_of, snapshot, _normwise

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(recipe, n, dk, dv, t0, steps, seed=0, edit=None):
    d = gen_steps(recipe, n, dk, dv, [seed], t0, steps, device="cpu")
    if edit is not None:
        edit(d)
    return {k: v.to(DEV) for k, v in d.items()}, {k: v.numpy() for k, v in d.items()}


def zero_directions(d, dk):
    """Inputs with no update direction in places: k columns that are exactly
    zero in every step and head (including a column inside the last lane's
    chunk and one on a group edge), and heads whose beta is zero (w = 0)."""
    for c in (0, 5, dk // 2, dk - 1):
        d["k"][:, :, c] = 0.0
    d["beta"][:, 1::3] = 0.0


def _np_step(d, t):
    return (d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t])


def _run_teacher_forced(cfg, steps, recipe, warmup=4, edit=None):
    """Run the GPU path, comparing each step with the oracle from the GPU's state."""
    ocfg = ocfg_of(cfg)
    st = lsq.LsqState(cfg, device=DEV).zero()
    rep = Report()
    t0 = 0
    if cfg.policy == lsq.POLICY_PERSISTENT:
        f = lsq.LsqState(lsq.LsqConfig(cfg.batch, cfg.heads, cfg.dk, cfg.dv, 32, 1,
                                       lsq.POLICY_NONE, 0, cfg.delta, cfg.decay), device=DEV).zero()
        dg, _ = _inputs(recipe, cfg.n, cfg.dk, cfg.dv, 0, warmup, edit=edit)
        f.run(dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"])
        st.calibrate(f.f32)
        # calibration itself: bit-exact against the oracle's quantiser
        want = oracle.calibrate(ocfg, f.f32.cpu().numpy())
        got = snapshot(st)
        assert np.array_equal(got.codes, want.codes)
        assert np.array_equal(got.scales, want.scales)
        t0 = warmup
    dg, dn = _inputs(recipe, cfg.n, cfg.dk, cfg.dv, t0, steps, edit=edit)
    before = snapshot(st)
    if cfg.rounding == lsq.ROUND_DITHER:
        st.step_index = 1000 + 37 * cfg.dk     # any position: the sequence is stateless
    for t in range(steps):
        ocfg_t = ocfg.replace(step=st.step_index)
        out = st.step(dg["q"][t], dg["k"][t], dg["v"][t], dg["alpha"][t], dg["beta"][t])
        o, o_ref = out if cfg.policy == lsq.POLICY_YOKED else (out, None)
        after = snapshot(st)
        rep.add(compare_step(ocfg_t, before, _np_step(dn, t), after, o.cpu().numpy(),
                             None if o_ref is None else o_ref.cpu().numpy()))
        before = after
    return rep


COMBOS = [(bits, dk, pol, rnd, dl, dc)
          for bits in (4, 8)
          for dk in (128, 64)
          for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT, lsq.POLICY_YOKED)
          for rnd in (lsq.ROUND_RNE, lsq.ROUND_BDR, lsq.ROUND_DITHER)
          for dl in (0, 1)
          for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,pol,rnd,dl,dc", COMBOS)
def test_step_matches_oracle(bits, dk, pol, rnd, dl, dc):
    group = 32 if bits == 4 else 64
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=44, bits=bits, group=min(group, dk),
                        policy=pol, rounding=rnd, delta=dl, decay=dc)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run_teacher_forced(cfg, steps=6, recipe=recipe)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


MULTI = [(bits, dk, pol, rnd, dl, dc)
         for bits in (4, 8)
        for dk in (128, 64)
        for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
        for rnd in (lsq.ROUND_RNE, lsq.ROUND_BDR)
        for dl in (0, 1)
        for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,pol,rnd,dl,dc", MULTI)
def test_multi_row_waves_match_oracle(bits, dk, pol, rnd, dl, dc):
    """States of 2048 heads: the launch shape of few-head states (4096 waves),
    two waves per head with four row-iterations each, so that every wave walks
    its rows with the next row's loads in flight and reloads its first buffer
    (the small states above take one row-iteration per wave).  Dv leaves a
    ragged last row-iteration."""
    group = 32 if bits == 4 else 64
    dv = 120 if dk == 128 else 250
    cfg = lsq.LsqConfig(batch=64, heads=32, dk=dk, dv=dv, bits=bits, group=min(group, dk),
                        policy=pol, rounding=rnd, delta=dl, decay=dc)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run_teacher_forced(cfg, steps=3, recipe=recipe)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


ZD = [(bits, dk, pol, dl, dc)
      for bits in (4, 8)
      for dk in (128, 64)
      for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
      for dl in (0, 1)
      for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,pol,dl,dc", ZD)
def test_bdr_without_update_direction(bits, dk, pol, dl, dc):
    """Directional rounding where the update has no sign (k_c = 0, or w = 0
    for a head with beta = 0): those elements round to nearest."""
    group = 32 if bits == 4 else 64
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=44, bits=bits, group=min(group, dk),
                        policy=pol, rounding=lsq.ROUND_BDR, delta=dl, decay=dc)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run_teacher_forced(cfg, steps=5, recipe=recipe,
                              edit=lambda d: zero_directions(d, dk))
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


def decays_near_one(d):
    """Decays at and around the head-level bound 1 - 2^-20 of the round-up
    candidate's range test: per head (h mod 5) exactly 1, 1 - 2^-21 (both
    tested row by row; at 1 the bound can fail and rows take the
    two-instruction clamp), 1 - 2^-20 (the largest decay the head-level test
    settles), 1 - 2^-19, and the recipe's own.  A diagonal decay puts the
    value on one column of the head and keeps the recipe's elsewhere."""
    a = d["alpha"]
    vals = (1.0, 1.0 - 2.0 ** -21, 1.0 - 2.0 ** -20, 1.0 - 2.0 ** -19)
    for i, v in enumerate(vals):
        if a.dim() == 2:
            a[:, i::5] = v
        else:
            a[:, i::5, 3] = v


NEAR1 = [(bits, dl, dc)
         for bits in (4, 8)
         for dl in (0, 1)
         for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dl,dc", NEAR1)
def test_bdr_decays_near_one(bits, dl, dc):
    """Frozen scales with directional rounding, decays at and near 1: the
    head-level and per-row range tests of the round-up candidate, and the
    general clamp where the test fails, all against the oracle bit for bit."""
    group = 32 if bits == 4 else 64
    cfg = lsq.LsqConfig(batch=2, heads=5, dk=128, dv=44, bits=bits, group=group,
                        policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_BDR, delta=dl, decay=dc)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run_teacher_forced(cfg, steps=6, recipe=recipe, edit=decays_near_one)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


G16 = [(bits, dk, pol, rnd, dc)
       for bits in (4, 8)
       for dk in (128, 64)
       for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT, lsq.POLICY_YOKED)
       for rnd in (lsq.ROUND_RNE, lsq.ROUND_BDR, lsq.ROUND_DITHER)
       for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,pol,rnd,dc", G16)
def test_group16_matches_oracle(bits, dk, pol, rnd, dc):
    """16-element groups: two groups inside each lane's 32 elements."""
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=44, bits=bits, group=16,
                        policy=pol, rounding=rnd, delta=1, decay=dc)
    rep = _run_teacher_forced(cfg, steps=5, recipe="gla" if dc == lsq.DECAY_DIAG else "gdn")
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


SF = [(bits, dk, pol, rnd, dl, dc, fmt)
      for bits in (4, 8)
      for dk in (128, 64)
      for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT, lsq.POLICY_YOKED)
      for rnd in (lsq.ROUND_RNE, lsq.ROUND_BDR)
      for dl in (0, 1)
      for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)
      for fmt in (lsq.SCALE_F16, lsq.SCALE_BF16)]


@pytest.mark.parametrize("bits,dk,pol,rnd,dl,dc,fmt", SF)
def test_16bit_scales_match_oracle(bits, dk, pol, rnd, dl, dc, fmt):
    """binary16 / bfloat16 stored scales: rounded on both sides before the codes
    are formed; calibration bit-exact, steps to the usual bar."""
    group = 32 if bits == 4 else 64
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=44, bits=bits, group=min(group, dk),
                        policy=pol, rounding=rnd, delta=dl, decay=dc, scale_fmt=fmt)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run_teacher_forced(cfg, steps=6, recipe=recipe)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


@pytest.mark.parametrize("bits,pol,rnd,fmt", [(b, p, r, f) for b in (4, 8)
                                              for p in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
                                              for r in (lsq.ROUND_RNE, lsq.ROUND_BDR, lsq.ROUND_DITHER)
                                              for f in (lsq.SCALE_F16, lsq.SCALE_BF16)])
def test_group16_16bit_scales_match_oracle(bits, pol, rnd, fmt):
    """16-element groups with 16-bit scales: both of a lane's scales in one dword."""
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=128, dv=44, bits=bits, group=16, policy=pol,
                        rounding=rnd, delta=1, decay=lsq.DECAY_DIAG, scale_fmt=fmt)
    rep = _run_teacher_forced(cfg, steps=5, recipe="gla")
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


ALT = [(bits, dk, rnd, dl, dc)
       for bits in (4, 8)
       for dk in (128, 64)
       for rnd in (lsq.ROUND_BDR_A, lsq.ROUND_BDR_B)
       for dl in (0, 1)
       for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,rnd,dl,dc", ALT)
def test_rejected_bdr_readings_match_oracle(bits, dk, rnd, dl, dc):
    """The two directional readings not taken (sensitivity flags), persistent scale."""
    group = 32 if bits == 4 else 64
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=44, bits=bits, group=min(group, dk),
                        policy=lsq.POLICY_PERSISTENT, rounding=rnd, delta=dl, decay=dc)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run_teacher_forced(cfg, steps=6, recipe=recipe)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)
    if rnd == lsq.ROUND_BDR_A:
        assert rep.bdr_fired == 0                     # equals RNE on a frozen grid


HEAD = [(bits, dk, pol, rnd, dl, dc)
        for bits in (4, 8)
        for dk in (128, 64)
        for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
        for rnd in (lsq.ROUND_RNE, lsq.ROUND_BDR)
        for dl in (0, 1)
        for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,pol,rnd,dl,dc", HEAD)
def test_head_scale_matches_oracle(bits, dk, pol, rnd, dl, dc):
    """One scale per head (group 0), Dv = 100."""
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=100, bits=bits, group=0, policy=pol,
                        rounding=rnd, delta=dl, decay=dc)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run_teacher_forced(cfg, steps=6, recipe=recipe)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


HEAD_DV = [(bits, dk, dv, rnd, dc)
           for bits, rnd, dc in ((4, lsq.ROUND_BDR, lsq.DECAY_SCALAR), (8, lsq.ROUND_RNE, lsq.DECAY_DIAG))
           for dk, dvs in ((128, (16, 128, 129, 200, 256, 257, 700)), (64, (256, 300, 512, 513)))
           for dv in dvs]


@pytest.mark.parametrize("bits,dk,dv,rnd,dc", HEAD_DV)
def test_dynamic_head_scale_heights(bits, dk, dv, rnd, dc):
    """Dynamic per-head scales over head heights on both sides of the kernel
    choice: rows held in registers by eight waves (up to 8 row-iterations) or
    sixteen (up to 16), else two passes."""
    cfg = lsq.LsqConfig(batch=1, heads=3, dk=dk, dv=dv, bits=bits, group=0,
                        policy=lsq.POLICY_DYNAMIC, rounding=rnd, delta=1, decay=dc)
    rep = _run_teacher_forced(cfg, steps=4, recipe="gla" if dc == lsq.DECAY_DIAG else "gdn")
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


def test_16bit_scale_buffers_are_half_size():
    for fmt, nbytes in ((lsq.SCALE_F32, 4), (lsq.SCALE_F16, 2), (lsq.SCALE_BF16, 2)):
        cfg = lsq.LsqConfig(batch=1, heads=2, dk=128, dv=16, bits=4, group=32, scale_fmt=fmt)
        st = lsq.LsqState(cfg, device=DEV)
        assert st.scales.element_size() == nbytes
        assert lsq.lsq_state_sizes(cfg)[1] == 2 * 16 * 4 * nbytes


@pytest.mark.parametrize("bits,group", [(4, 64), (4, 128), (8, 32), (8, 128)])
def test_other_group_sizes(bits, group):
    for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT):
        cfg = lsq.LsqConfig(batch=1, heads=5, dk=128, dv=24, bits=bits, group=group, policy=pol,
                            rounding=lsq.ROUND_BDR, delta=1, decay=0)
        rep = _run_teacher_forced(cfg, steps=4, recipe="gdn")
        assert rep.ok, str(rep)


@pytest.mark.parametrize("dk", [128, 64])
@pytest.mark.parametrize("dl,dc", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_fp32_state_free_running(dk, dl, dc):
    """Unquantised mode over a whole horizon: S_H and every o_t within 1e-5."""
    cfg = lsq.LsqConfig(batch=3, heads=2, dk=dk, dv=37, bits=32, group=1,
                        policy=lsq.POLICY_NONE, rounding=0, delta=dl, decay=dc)
    H = 40
    recipe = "gla" if dc else ("gdn" if dl else "mamba2")
    dg, dn = _inputs(recipe, cfg.n, dk, cfg.dv, 0, H)
    st = lsq.LsqState(cfg, device=DEV).zero()
    o = st.run(dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"])
    ost = oracle.zero_state(ocfg_of(cfg))
    oo, _ = oracle.run(ocfg_of(cfg), ost, dn["q"], dn["k"], dn["v"], dn["alpha"], dn["beta"])
    assert _normwise(st.f32.cpu().numpy(), ost.f32) <= 1e-5
    for t in range(H):
        assert _normwise(o[t].cpu().numpy(), oo[t]) <= 1e-5, t


def test_run_equals_repeated_steps_and_is_deterministic():
    cfg = lsq.LsqConfig(batch=4, heads=4, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_DYNAMIC, rounding=lsq.ROUND_BDR, delta=1, decay=0)
    dg, _ = _inputs("gdn", cfg.n, 128, 128, 0, 10)
    a = lsq.LsqState(cfg, device=DEV).zero()
    b = lsq.LsqState(cfg, device=DEV).zero()
    c = lsq.LsqState(cfg, device=DEV).zero()
    oa = a.run(dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"])
    ob = torch.stack([b.step(dg["q"][t], dg["k"][t], dg["v"][t], dg["alpha"][t], dg["beta"][t])
                      for t in range(10)])
    oc = c.run(dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"])
    for x, y in ((a, b), (a, c)):
        assert torch.equal(x.codes, y.codes) and torch.equal(x.scales, y.scales)
    assert torch.equal(oa, ob) and torch.equal(oa, oc)


def test_dither_step_index_drives_the_sequence():
    """The step index advances per step and per run; restoring it resumes the
    same dithered trajectory; the same state at another index differs."""
    cfg = lsq.LsqConfig(batch=2, heads=4, dk=128, dv=64, bits=4, group=32,
                        policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_DITHER, delta=1, decay=0)
    dg, _ = _inputs("gdn", cfg.n, 128, 64, 0, 8)
    S0 = torch.randn(cfg.n, 64, 128, device=DEV) * 0.1
    a = lsq.LsqState(cfg, device=DEV).zero().calibrate(S0)
    b = lsq.LsqState(cfg, device=DEV).zero().calibrate(S0)
    assert a.step_index == 0
    oa = a.run(*(dg[x] for x in ("q", "k", "v", "alpha", "beta")))
    assert a.step_index == 8
    ob = torch.stack([b.step(*(dg[x][t] for x in ("q", "k", "v", "alpha", "beta"))) for t in range(8)])
    assert b.step_index == 8
    assert torch.equal(oa, ob) and torch.equal(a.codes, b.codes)
    c = lsq.LsqState(cfg, device=DEV).zero().calibrate(S0)
    c.step_index = 5
    c.step(*(dg[x][0] for x in ("q", "k", "v", "alpha", "beta")))
    d = lsq.LsqState(cfg, device=DEV).zero().calibrate(S0)
    d.step(*(dg[x][0] for x in ("q", "k", "v", "alpha", "beta")))
    assert not torch.equal(c.codes, d.codes)
    with pytest.raises(lsq.LsqError, match="INVALID_ARG"):
        c.step_index = -1


def test_checkpoint_resume_is_bit_identical():
    """A copy of the state buffers bound to a new handle resumes exactly."""
    cfg = lsq.LsqConfig(batch=2, heads=8, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_BDR, delta=1, decay=0)
    dg, _ = _inputs("gdn", cfg.n, 128, 128, 0, 12)
    S0 = torch.randn(cfg.n, 128, 128, device=DEV) * 0.1
    a = lsq.LsqState(cfg, device=DEV).zero().calibrate(S0)
    a.run(*(dg[x][:6] for x in ("q", "k", "v", "alpha", "beta")))
    b = lsq.LsqState(cfg, device=DEV)
    b.codes.copy_(a.codes)
    b.scales.copy_(a.scales)
    with pytest.raises(lsq.LsqError, match="NOT_CALIBRATED"):
        b.step(dg["q"][6], dg["k"][6], dg["v"][6], dg["alpha"][6], dg["beta"][6])
    b.set_calibrated(True)
    oa = a.run(*(dg[x][6:] for x in ("q", "k", "v", "alpha", "beta")))
    ob = b.run(*(dg[x][6:] for x in ("q", "k", "v", "alpha", "beta")))
    assert torch.equal(oa, ob) and torch.equal(a.codes, b.codes)


def test_edge_cases():
    # empty batch: steps are no-ops
    cfg = lsq.LsqConfig(batch=0, heads=4, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_DYNAMIC)
    st = lsq.LsqState(cfg, device=DEV).zero()
    z = torch.zeros(0, 128, device=DEV)
    st.step(z, z, z, torch.zeros(0, device=DEV), torch.zeros(0, device=DEV))
    # a single row, one group spanning the whole row, zero inputs keep S = 0
    cfg = lsq.LsqConfig(batch=1, heads=3, dk=128, dv=1, bits=8, group=128,
                        policy=lsq.POLICY_DYNAMIC, rounding=lsq.ROUND_BDR, delta=1)
    st = lsq.LsqState(cfg, device=DEV).zero()
    zq = torch.zeros(3, 128, device=DEV)
    o = st.step(zq, zq, torch.zeros(3, 1, device=DEV), torch.ones(3, device=DEV),
                torch.ones(3, device=DEV))
    assert torch.count_nonzero(st.codes) == 0 and torch.count_nonzero(o) == 0
    assert torch.count_nonzero(st.scales) == 0
    # saturation: a persistent scale far too small clamps every written element
    cfg = lsq.LsqConfig(batch=1, heads=2, dk=128, dv=16, bits=4, group=32,
                        policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_BDR, delta=0)
    st = lsq.LsqState(cfg, device=DEV).zero()
    st.calibrate(torch.full((2, 16, 128), 1e-6, device=DEV))
    k = torch.ones(2, 128, device=DEV)
    st.step(k, k, torch.full((2, 16), 1e3, device=DEV), torch.ones(2, device=DEV),
            torch.ones(2, device=DEV))
    codes = oracle.unpack(st.codes.cpu().numpy(), 4, 128)
    assert np.all(codes == 7)


DQ = [(bits, dk, group, fmt)
      for bits in (4, 8)
      for dk in (128, 64)
      for group in (0, 16, 32, 64)
      for fmt in (0, 1, 2)
      if not (group == 0 and fmt)]


@pytest.mark.parametrize("bits,dk,group,fmt", DQ)
def test_dequantize_matches_oracle(bits, dk, group, fmt):
    """lsq_state_dequantize: fl(C s) bit for bit against the oracle's, after a few
    dynamic steps (per-head scales: persistent, calibrated), ragged Dv."""
    pol = lsq.POLICY_PERSISTENT if group == 0 else lsq.POLICY_DYNAMIC
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=37, bits=bits, group=group,
                        policy=pol, rounding=lsq.ROUND_BDR, delta=1, scale_fmt=fmt)
    try:
        lsq.lsq_state_sizes(cfg)
    except lsq.LsqError:
        pytest.skip(f"not supported: {cfg}")
    st = lsq.LsqState(cfg, device=DEV).zero()
    if pol == lsq.POLICY_PERSISTENT:
        g = torch.Generator(device=DEV).manual_seed(3)
        st.calibrate(torch.randn(cfg.n, cfg.dv, cfg.dk, device=DEV, generator=g) * 0.2)
    dg, _ = _inputs("gdn", cfg.n, cfg.dk, cfg.dv, 0, 3)
    for t in range(3):
        st.step(dg["q"][t], dg["k"][t], dg["v"][t], dg["alpha"][t], dg["beta"][t])
    got = st.dequantize().cpu().numpy()
    want = oracle.dequantize(ocfg_of(cfg), snapshot(st))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.count_nonzero(got) > 0


def test_dequantize_fp32_state_is_a_copy():
    cfg = lsq.LsqConfig(batch=1, heads=2, dk=64, dv=9, bits=32, group=32, policy=lsq.POLICY_NONE)
    st = lsq.LsqState(cfg, device=DEV).zero()
    S = torch.randn(cfg.n, cfg.dv, cfg.dk, device=DEV)
    st.calibrate(S)
    assert torch.equal(st.dequantize(), S)


FREE = [(bits, pol, rnd, dc, dk)
        for bits in (4, 8)
        for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT, lsq.POLICY_YOKED)
        for rnd in (lsq.ROUND_RNE, lsq.ROUND_BDR, lsq.ROUND_DITHER)
        for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)
        for dk in (128, 64)]


@pytest.mark.parametrize("bits,pol,rnd,dc,dk", FREE)
def test_free_running_bit_exact(bits, pol, rnd, dc, dk):
    """Free-running GPU and oracle trajectories from the same start, 256 steps of
    Gated DeltaNet inputs with no teacher forcing: with every operation of the
    step fixed on both sides (the row dots' summation order included), the two
    trajectories stay identical: codes and scales after the horizon, and the
    output of every step."""
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=48, bits=bits, group=32 if bits == 4 else 64,
                        policy=pol, rounding=rnd, delta=1, decay=dc)
    H = 256
    st = lsq.LsqState(cfg, device=DEV).zero()
    ost = oracle.zero_state(ocfg_of(cfg))
    if pol == lsq.POLICY_PERSISTENT:
        g = torch.Generator(device=DEV).manual_seed(7)
        S0 = torch.randn(cfg.n, cfg.dv, cfg.dk, device=DEV, generator=g) * 0.3
        st.calibrate(S0)
        ost = oracle.calibrate(ocfg_of(cfg), S0.cpu().numpy())
    recipe = "gla" if dc == lsq.DECAY_DIAG else "gdn"
    dg, dn = _inputs(recipe, cfg.n, cfg.dk, cfg.dv, 0, H)
    out = st.run(dg["q"], dg["k"], dg["v"], dg["alpha"], dg["beta"])
    o = (out[0] if pol == lsq.POLICY_YOKED else out).cpu().numpy()
    ow, _ = oracle.run(ocfg_of(cfg), ost, dn["q"], dn["k"], dn["v"], dn["alpha"], dn["beta"])
    got = snapshot(st)
    assert np.array_equal(got.codes, ost.codes)
    assert np.array_equal(got.scales, ost.scales)
    if pol == lsq.POLICY_YOKED:
        assert np.array_equal(got.ref, ost.ref)
    assert np.array_equal(o.view(np.uint32), ow.view(np.uint32))
