"""GPU parity of the Low-Rank Bypass step against the CPU oracle.

Teacher-forced as the plain step (tests/parity.py): before every step the
oracle takes the GPU's codes, scales and bypass slots (a, and the b copy the
step reads); after it the codes, scales and o are held to the usual bar, and
the slots the next step will read are compared bit for bit: decayed slots, the
new b = k and the new a = w (the delta projection is summed in the one order
both sides fix).  Runs of 2r+1 steps cover two merges and the slot reuse after
a merge.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_recurrent_state_amd as lsq
from quantized_recurrent_state_amd.inputs import gen_steps
from tests.parity import Report, compare_step, ocfg_of, snapshot

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(recipe, n, dk, dv, steps, seed=4, edit=None):
    d = gen_steps(recipe, n, dk, dv, [seed], 0, steps, device="cpu")
    if edit is not None:
        edit(d)
    return {k: v.to(DEV) for k, v in d.items()}, {k: v.numpy() for k, v in d.items()}


def _run(cfg, steps, recipe, t0=0, edit=None):
    R = cfg.lrb_rank
    st = lsq.LsqState(cfg, device=DEV).zero()
    if cfg.policy == lsq.POLICY_PERSISTENT:
        g = torch.Generator(device=DEV).manual_seed(1)
        st.calibrate(torch.randn(cfg.n, cfg.dv, cfg.dk, device=DEV, generator=g) * 0.3)
    st.step_index = t0
    dg, dn = _inputs(recipe, cfg.n, cfg.dk, cfg.dv, steps, edit=edit)
    rep = Report()
    diag = cfg.decay == lsq.DECAY_DIAG
    for t in range(steps):
        ti = st.step_index
        before = snapshot(st)
        before.lrb_a = st.lrb_a.cpu().numpy().copy()
        before.lrb_b = st.lrb_b[:, (ti & 1) if diag else 0].cpu().numpy().copy()
        o = st.step(dg["q"][t], dg["k"][t], dg["v"][t], dg["alpha"][t], dg["beta"][t])
        after = snapshot(st)
        ora = []
        rep.add(compare_step(ocfg_of(cfg, step=ti).replace(lrb_rank=R), before,
                             tuple(dn[x][t] for x in ("q", "k", "v", "alpha", "beta")), after,
                             o.cpu().numpy(), oracle_after=ora))
        n_after = (ti + 1) % R
        if n_after:
            want = ora[0]
            ga = st.lrb_a.cpu().numpy()
            gb = st.lrb_b[:, ((ti + 1) & 1) if diag else 0].cpu().numpy()
            used = n_after - 1                     # slots decayed this step
            assert np.array_equal(ga[:, :used], want.lrb_a[:, :used]), (t, "decayed a")
            assert np.array_equal(gb[:, :n_after], want.lrb_b[:, :n_after]), (t, "b")
            assert np.array_equal(ga[:, used], want.lrb_a[:, used]), (t, "new a")
    return rep


COMBOS = [(bits, dk, pol, rnd, dl, dc)
          for bits in (4, 8)
          for dk in (128, 64)
          for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
          for rnd in (lsq.ROUND_RNE, lsq.ROUND_BDR, lsq.ROUND_DITHER)
          for dl in (0, 1)
          for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,pol,rnd,dl,dc", COMBOS)
def test_bypass_step_matches_oracle(bits, dk, pol, rnd, dl, dc):
    R = 3
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=dk, dv=44, bits=bits, group=min(32 if bits == 4 else 64, dk),
                        policy=pol, rounding=rnd, delta=dl, decay=dc, lrb_rank=R)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run(cfg, 2 * R + 1, recipe)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


@pytest.mark.parametrize("R", [1, 2, 8])
def test_bypass_ranks_and_offsets(R):
    cfg = lsq.LsqConfig(batch=4, heads=4, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_BDR, delta=1,
                        decay=lsq.DECAY_SCALAR, lrb_rank=R)
    rep = _run(cfg, R + 3, "gdn", t0=5 * R + 1)     # start mid-period
    assert rep.ok, str(rep)


@pytest.mark.parametrize("bits,pol,dl,dc", [(b, p, dl, dc) for b in (4, 8)
                                            for p in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
                                            for dl in (0, 1)
                                            for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)])
def test_bypass_merge_without_update_direction(bits, pol, dl, dc):
    """Merges where the buffer's value U is exactly zero (k columns zero in
    every step, heads with beta = 0): those elements round to nearest."""
    from tests.test_gpu_parity import zero_directions
    R = 3
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=128, dv=44, bits=bits, group=32 if bits == 4 else 64,
                        policy=pol, rounding=lsq.ROUND_BDR, delta=dl, decay=dc, lrb_rank=R)
    recipe = "gla" if dc == lsq.DECAY_DIAG else ("gdn" if dl else "mamba2")
    rep = _run(cfg, 2 * R + 1, recipe, edit=lambda d: zero_directions(d, 128))
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


@pytest.mark.parametrize("R,bits,pol,rnd,dc", [
    (5, 4, lsq.POLICY_DYNAMIC, lsq.ROUND_BDR, lsq.DECAY_DIAG),
    (6, 8, lsq.POLICY_DYNAMIC, lsq.ROUND_RNE, lsq.DECAY_SCALAR),
    (7, 8, lsq.POLICY_PERSISTENT, lsq.ROUND_BDR, lsq.DECAY_SCALAR),
    (5, 4, lsq.POLICY_PERSISTENT, lsq.ROUND_DITHER, lsq.DECAY_DIAG),
])
def test_bypass_large_ranks(R, bits, pol, rnd, dc):
    """Ranks 5 to 8 take their own kernel instances: other flags than the rank-8 case above."""
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=128, dv=44, bits=bits, group=32 if bits == 4 else 64,
                        policy=pol, rounding=rnd, delta=1, decay=dc, lrb_rank=R)
    rep = _run(cfg, R + 2, "gla" if dc == lsq.DECAY_DIAG else "gdn", t0=2 * R - 1)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)
