"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same handles, same launch geometry, same device-generated
inputs), on sampled heads compared teacher-forced with the CPU oracle.

  la       1 head, 64x64 INT8 g64 dynamic: every head, the whole 256-step horizon
  gla      1024 heads, INT4 g32 persistent, diagonal decay: fp32 warmup and
           calibration checked, then the whole 1024-step horizon on sampled heads
  gdn      4096 heads, delta rule, dynamic vs yoked INT4 g32 on identical inputs:
           2048 steps, checked at sampled steps
  mamba2   8192 heads, Dv 64, INT8 g64 persistent, BDR vs RNE: 4096 steps,
           checked at sampled steps
  stack24  393216 heads in two launches (INT8 g64 layers 0-3, INT4 g32 layers
           4-23), persistent, BDR: warmup, calibration and the whole 32768-step
           horizon checked at sampled steps (the first four, every 4096th, the
           last); the first steps of the stack's variants the benchmark runs
           (RNE, Weyl dither, 16-element groups, bfloat16 scales, one scale per
           head, reading B'), and of Gated DeltaNet with a dynamic scale per head
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_recurrent_state_amd as lsq
from quantized_recurrent_state_amd import runner
from quantized_recurrent_state_amd.inputs import WORKLOADS
from tests.parity import Report, compare_step, ocfg_of, snapshot

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _sample(n, m):
    return torch.as_tensor(np.unique(np.linspace(0, n - 1, min(n, m)).astype(np.int64)), device=DEV)


def _check_calibration(st, S_W, sel):
    """The persistent scales and codes equal the oracle's quantiser on S_W."""
    ocfg = ocfg_of(st.cfg).replace(batch=len(sel), heads=1)
    want = oracle.calibrate(ocfg, S_W.index_select(0, sel).cpu().numpy())
    got = snapshot(st, heads=sel)
    assert np.array_equal(got.codes, want.codes)
    assert np.array_equal(got.scales, want.scales)


def _run_checked(wl, arms_state, t_first, steps, check_steps, sel_n, chunk=64, per_step=None,
                 progress=0):
    """Step every arm through `steps` steps; at the steps in check_steps compare
    the sampled heads teacher-forced.  Returns one Report per arm; per_step, if
    given, collects (step, arm index, Report) of every check."""
    reps = [Report() for _ in arms_state]
    sels = [_sample(st.cfg.n, sel_n) for st in arms_state]
    npl = wl.batch * wl.heads
    shared = None
    for c0 in range(0, steps, chunk):
        nc = min(chunk, steps - c0)
        inputs = []
        for arm in wl.arms:
            if wl.shared_inputs and shared is not None and shared[0] == c0:
                inputs.append(shared[1])
                continue
            d = runner.inputs(wl, arm, t_first + c0, nc, npl, DEV)
            inputs.append(d)
            if wl.shared_inputs:
                shared = (c0, d)
        for j in range(nc):
            t = c0 + j
            for ai, st in enumerate(arms_state):
                d = inputs[ai]
                chk = t in check_steps
                if chk:
                    before = snapshot(st, heads=sels[ai])
                    step_index = st.step_index          # the dither's (and the bypass's) position
                    if st.cfg.lrb_rank > 0:             # the bypass slots this step reads
                        cin = (step_index & 1) if st.cfg.decay == lsq.DECAY_DIAG else 0
                        before.lrb_a = st.lrb_a.index_select(0, sels[ai]).cpu().numpy().copy()
                        before.lrb_b = st.lrb_b[:, cin].index_select(0, sels[ai]).cpu().numpy().copy()
                out = st.step(d["q"][j], d["k"][j], d["v"][j], d["alpha"][j], d["beta"][j])
                if chk:
                    o, o_ref = out if st.cfg.policy == lsq.POLICY_YOKED else (out, None)
                    sel = sels[ai]
                    after = snapshot(st, heads=sel)
                    inp = tuple(d[x][j].index_select(0, sel).cpu().numpy()
                                for x in ("q", "k", "v", "alpha", "beta"))
                    ocfg = ocfg_of(st.cfg, step=step_index).replace(batch=len(sel), heads=1,
                                                                    lrb_rank=st.cfg.lrb_rank)
                    r1 = compare_step(
                        ocfg, before, inp, after, o.index_select(0, sel).cpu().numpy(),
                        None if o_ref is None else o_ref.index_select(0, sel).cpu().numpy())
                    reps[ai].add(r1)
                    if per_step is not None:
                        per_step.append((t, ai, r1))
        del inputs
        if progress and (c0 + nc) // progress != c0 // progress:
            print(f"{wl.name}: {c0 + nc} of {steps} steps", flush=True)
    return reps


def _prepare(wl, check_cal=True, sel_n=32):
    states, t_first = [], 0
    for arm in wl.arms:
        st, t_first, S_W = runner.prepare(wl, arm, DEV, keep_fp32=True)
        if S_W is not None and check_cal:
            _check_calibration(st, S_W, _sample(st.cfg.n, sel_n))
        del S_W
        states.append(st)
    torch.cuda.empty_cache()
    return states, t_first


def _assert_ok(wl, reps):
    for arm, rep in zip(wl.arms, reps):
        print(f"\n{wl.name} / {arm.name}: {rep}")
        assert rep.codes > 0
        assert rep.ok, f"{arm.name}: {rep}"
        assert rep.failed == 0 and rep.o_differ == 0, f"{arm.name}: {rep}"


def test_la_whole_horizon():
    wl = WORKLOADS["la"]
    states, t0 = _prepare(wl)
    reps = _run_checked(wl, states, t0, wl.steps, set(range(wl.steps)), sel_n=1)
    _assert_ok(wl, reps)


def test_gla_whole_horizon_sampled_heads():
    wl = WORKLOADS["gla"]
    states, t0 = _prepare(wl)
    reps = _run_checked(wl, states, t0, wl.steps, set(range(wl.steps)), sel_n=24, chunk=128)
    _assert_ok(wl, reps)


def test_gdn_dynamic_vs_yoked():
    wl = WORKLOADS["gdn"]
    states, t0 = _prepare(wl)
    checks = set(range(8)) | set(range(255, wl.steps, 256))
    reps = _run_checked(wl, states, t0, wl.steps, checks, sel_n=16, chunk=128)
    _assert_ok(wl, reps)


def test_mamba2_bdr_vs_rne():
    wl = WORKLOADS["mamba2"]
    states, t0 = _prepare(wl)
    checks = set(range(4)) | set(range(511, wl.steps, 512))
    reps = _run_checked(wl, states, t0, wl.steps, checks, sel_n=16, chunk=128)
    _assert_ok(wl, reps)
    # the two arms ran on identical inputs from identical calibrated states
    assert reps[0].bdr_fired > 0 and reps[1].bdr_fired == 0


@pytest.mark.timeout(1200)
def test_stack24_whole_horizon():
    """The 24-layer stack (393 216 heads, INT8 g64 layers 0-3 and INT4 g32 layers
    4-23, persistent scales, BDR, delta rule) through all 32 768 quantised steps
    after its 64-step fp32 warmup, in the benchmark's launch configuration:
    teacher-forced on 48 sampled heads per arm at steps 0-3, every 4096th step
    and the last one; clamp and directional-rounding rates reported along the
    horizon ("When Dynamic Scaling Fails", abstract: group-wise INT4 run out to
    32K)."""
    wl = WORKLOADS["stack24"]
    states, t0 = _prepare(wl, sel_n=48)
    checks = set(range(4)) | set(range(4095, wl.steps, 4096)) | {wl.steps - 1}
    per_step = []
    reps = _run_checked(wl, states, t0, wl.steps, checks, sel_n=48, chunk=32, per_step=per_step,
                        progress=4096)
    for t, ai, r1 in per_step:
        n = max(1, r1.codes)
        print(f"step {t:5d} {wl.arms[ai].name}: clamp rate {r1.clamped / n:.5f} "
              f"directional-rounding rate {r1.bdr_fired / n:.5f} {'ok' if r1.ok else 'FAIL'}")
    assert {t for t, _, _ in per_step} == checks
    _assert_ok(wl, reps)
    del states
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", ["stack24", "stack24-rne", "stack24-dither", "stack24-g16",
                                 "stack24-bf16", "stack24-g16-bf16", "stack24-head", "stack24-bdrb",
                                 "stack24-lrb4", "gdn-head"])
def test_full_size_first_steps(key):
    wl = WORKLOADS[key]
    states, t0 = _prepare(wl, sel_n=48)
    reps = _run_checked(wl, states, t0, 6, set(range(6)), sel_n=48, chunk=6)
    _assert_ok(wl, reps)
    del states
    torch.cuda.empty_cache()
