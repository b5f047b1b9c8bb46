"""Seeded random sweep of configurations against the oracle (teacher-forced).

Draws bits, Dk, Dv (1 to 200, ragged against the rows a wave covers), heads,
group (16 to Dk, or one per head), scale policy, rounding (RNE, BDR, dither,
the two rejected readings), delta rule, decay and scale format, repaired into
combinations the library runs (a configuration it refuses is skipped on its
own status code); each runs a few steps against the oracle to the decode bar.
The bypass sweep uses the bypass harness (slots compared every step).
LSQ_RANDOM_SEEDS widens the decode sweep (default 80 seeds; the bypass sweep
takes a fifth as many).
"""
import os

import numpy as np
import pytest

import quantized_recurrent_state_amd as lsq
from tests.test_gpu_parity import _run_teacher_forced
from tests import test_gpu_lrb

N_SEEDS = int(os.environ.get("LSQ_RANDOM_SEEDS", "80"))

pytestmark = pytest.mark.gpu


def _draw(seed):
    """A random configuration, repaired into a combination the library runs."""
    rng = np.random.default_rng(1000 + seed)
    bits = int(rng.choice([4, 8]))
    dk = int(rng.choice([64, 128]))
    dv = int(rng.integers(1, 201))
    group = int(rng.choice([0, 16, 32, 64, dk]))
    policy = int(rng.choice([lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT, lsq.POLICY_YOKED]))
    rounding = int(rng.choice([lsq.ROUND_RNE, lsq.ROUND_BDR, lsq.ROUND_DITHER, lsq.ROUND_BDR_A,
                               lsq.ROUND_BDR_B]))
    scale_fmt = int(rng.choice([0, 0, 1, 2]))
    if rounding in (lsq.ROUND_BDR_A, lsq.ROUND_BDR_B):   # stored-code readings: frozen scale
        policy, group, scale_fmt = lsq.POLICY_PERSISTENT, max(group, 32), 0
    if group == 0:                                       # one scale per head
        policy = min(policy, lsq.POLICY_PERSISTENT)
        rounding = rounding if rounding in (lsq.ROUND_RNE, lsq.ROUND_BDR) else lsq.ROUND_BDR
        scale_fmt = 0
    return lsq.LsqConfig(batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 4)), dk=dk, dv=dv,
                         bits=bits, group=group, policy=policy, rounding=rounding,
                         delta=int(rng.integers(0, 2)), decay=int(rng.integers(0, 2)),
                         scale_fmt=scale_fmt)


@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_random_configuration(seed):
    cfg = _draw(seed)
    try:
        lsq.lsq_state_sizes(cfg)
    except lsq.LsqError as e:
        assert e.status in (1, 2)
        pytest.skip(f"not supported: {cfg}")
    recipe = "gla" if cfg.decay == lsq.DECAY_DIAG else ("gdn" if cfg.delta else "mamba2")
    rep = _run_teacher_forced(cfg, steps=4, recipe=recipe)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)


def _draw_bypass(seed):
    rng = np.random.default_rng(50000 + seed)
    bits = int(rng.choice([4, 8]))
    dk = int(rng.choice([64, 128]))
    R = int(rng.integers(1, 9))
    group = int(rng.choice([32, 64, dk])) if bits == 4 else int(rng.choice([64, dk]))
    cfg = lsq.LsqConfig(batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 4)), dk=dk,
                        dv=int(rng.integers(1, 160)), bits=bits, group=group,
                        policy=int(rng.choice([lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT])),
                        rounding=int(rng.choice([lsq.ROUND_RNE, lsq.ROUND_BDR, lsq.ROUND_DITHER])),
                        delta=int(rng.integers(0, 2)), decay=int(rng.integers(0, 2)), lrb_rank=R)
    return cfg, int(rng.integers(0, 3 * R))


@pytest.mark.parametrize("seed", range(max(1, N_SEEDS // 5)))
def test_random_bypass_configuration(seed):
    """Random rank (1 to 8), shape and flags of the bypass, started at a random phase."""
    cfg, t0 = _draw_bypass(seed)
    recipe = "gla" if cfg.decay == lsq.DECAY_DIAG else ("gdn" if cfg.delta else "mamba2")
    rep = test_gpu_lrb._run(cfg, 2 * cfg.lrb_rank + 1, recipe, t0=t0)
    print(f"\n{cfg}: {rep}")
    assert rep.ok, str(rep)
    assert rep.failed == 0 and rep.o_differ == 0, str(rep)
