"""GPU parity of the chunkwise prefill (lsq_prefill) against the CPU oracle.

Every operation of the state pass is fixed operation by operation (INT8
operand codes by round-half-even with the block's absmax scale, an exact
integer product, H = fl(h fl(s_V s_K)), one fma with gamma^C, the state's
own round-half-even requantisation), so the codes and scales are held bit for
bit, free-running over every chunk of the prompt, not teacher-forced.
Cases: INT4/INT8, Dk and Dv 64/128, dynamic and persistent scales, scalar and
diagonal decay, prompts that end mid-chunk, single tokens, the group sizes,
binary16 and bfloat16 scales, one scale per head,
a prompt split over several calls, a decode step after a prefill, and the
full-size workload (batch 64 x 16 heads, 4096 tokens) on sampled heads.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_recurrent_state_amd as lsq
from quantized_recurrent_state_amd.inputs import PREFILL_WORKLOADS, gen_steps
from tests.parity import compare_step, ocfg_of, snapshot

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _recipe(decay):
    return "gla" if decay == lsq.DECAY_DIAG else "la"


def _inputs(recipe, n, dk, dv, T, seed=11, t0=0):
    d = gen_steps(recipe, n, dk, dv, [seed], t0, T, device="cpu")
    return {k: v.to(DEV) for k, v in d.items()}, {k: v.numpy() for k, v in d.items()}


def _state(cfg, start_scale=0.05, seed=3):
    """A handle with a non-zero calibrated start state (persistent scales come from it)."""
    st = lsq.LsqState(cfg, device=DEV).zero()
    if start_scale:
        g = torch.Generator(device=DEV).manual_seed(seed)
        st.calibrate(torch.randn(cfg.n, cfg.dv, cfg.dk, device=DEV, generator=g) * start_scale)
    return st


def _check(cfg, st, before, dn, what=""):
    """Run the oracle over the same prompt from the GPU's start state; compare bit for bit."""
    ocfg = ocfg_of(cfg)
    want = before.copy()
    oracle.prefill(ocfg, want, dn["k"], dn["v"], dn["alpha"], dn["beta"], chunk=64)
    got = snapshot(st)
    nd = int((got.codes != want.codes).sum())
    assert nd == 0, f"{what}: {nd} of {want.codes.size} codes differ, first at " \
                    f"{np.argwhere(got.codes != want.codes)[:3].tolist()}"
    assert np.array_equal(got.scales, want.scales), f"{what}: scales differ"
    return want


COMBOS = [(bits, dk, dv, pol, dc)
          for bits in (4, 8)
          for dk in (128, 64)
          for dv in (128, 64)
          for pol in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
          for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)]


@pytest.mark.parametrize("bits,dk,dv,pol,dc", COMBOS)
def test_prefill_matches_oracle(bits, dk, dv, pol, dc):
    group = min(32 if bits == 4 else 64, dk)
    cfg = lsq.LsqConfig(batch=1, heads=3, dk=dk, dv=dv, bits=bits, group=group, policy=pol,
                        delta=0, decay=dc)
    T = 150                                     # two full chunks and a ragged one of 22
    st = _state(cfg)
    before = snapshot(st)
    dg, dn = _inputs(_recipe(dc), cfg.n, dk, dv, T)
    st.prefill(dg["k"], dg["v"], dg["alpha"], dg["beta"])
    torch.cuda.synchronize()
    _check(cfg, st, before, dn, str(cfg))
    assert st.step_index == T


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 128, 129])
def test_prefill_chunk_edges(T):
    cfg = lsq.LsqConfig(batch=2, heads=2, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_DYNAMIC, delta=0, decay=lsq.DECAY_DIAG)
    st = _state(cfg)
    before = snapshot(st)
    dg, dn = _inputs("gla", cfg.n, cfg.dk, cfg.dv, T, seed=5)
    st.prefill(dg["k"], dg["v"], dg["alpha"], dg["beta"])
    torch.cuda.synchronize()
    _check(cfg, st, before, dn, f"T={T}")


@pytest.mark.parametrize("bits,group", [(4, 16), (4, 64), (4, 128), (8, 16), (8, 32), (8, 128)])
def test_prefill_group_sizes(bits, group):
    cfg = lsq.LsqConfig(batch=1, heads=2, dk=128, dv=64, bits=bits, group=group,
                        policy=lsq.POLICY_DYNAMIC, delta=0, decay=lsq.DECAY_SCALAR)
    st = _state(cfg)
    before = snapshot(st)
    dg, dn = _inputs("mamba2", cfg.n, cfg.dk, cfg.dv, 100, seed=9)
    st.prefill(dg["k"], dg["v"], dg["alpha"], dg["beta"])
    torch.cuda.synchronize()
    _check(cfg, st, before, dn, f"bits={bits} g={group}")


@pytest.mark.parametrize("bits,pol,fmt,dc,group", [
    (b, p, f, dc, 32 if b == 4 else 64)
    for b in (4, 8)
    for p in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
    for f in (lsq.SCALE_F16, lsq.SCALE_BF16)
    for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)] + [
    (4, lsq.POLICY_DYNAMIC, lsq.SCALE_BF16, lsq.DECAY_DIAG, 16),
    (8, lsq.POLICY_DYNAMIC, lsq.SCALE_F16, lsq.DECAY_SCALAR, 128)])
def test_prefill_16bit_scales(bits, pol, fmt, dc, group):
    """binary16 and bfloat16 group scales: a dynamic scale is rounded to the
    stored format at every chunk before the codes are formed, a persistent one
    is read in the format; codes and stored scales bit for bit."""
    cfg = lsq.LsqConfig(batch=1, heads=3, dk=128, dv=128, bits=bits, group=group, policy=pol,
                        delta=0, decay=dc, scale_fmt=fmt)
    st = _state(cfg)
    before = snapshot(st)
    dg, dn = _inputs(_recipe(dc), cfg.n, cfg.dk, cfg.dv, 150, seed=13)
    st.prefill(dg["k"], dg["v"], dg["alpha"], dg["beta"])
    torch.cuda.synchronize()
    _check(cfg, st, before, dn, str(cfg))


@pytest.mark.parametrize("bits,pol,dc", [
    (b, p, dc)
    for b in (4, 8)
    for p in (lsq.POLICY_DYNAMIC, lsq.POLICY_PERSISTENT)
    for dc in (lsq.DECAY_SCALAR, lsq.DECAY_DIAG)])
def test_prefill_one_scale_per_head(bits, pol, dc):
    """group 0: a dynamic head scale is taken over all of the head's X at every
    chunk (the state waves meet at one more barrier), a frozen one is kept;
    codes and scales bit for bit, then a decode step from the prefilled state."""
    for dk, dv in ((128, 128), (64, 64)):
        cfg = lsq.LsqConfig(batch=1, heads=3, dk=dk, dv=dv, bits=bits, group=0, policy=pol,
                            delta=0, decay=dc)
        st = _state(cfg)
        before = snapshot(st)
        dg, dn = _inputs(_recipe(dc), cfg.n, dk, dv, 150, seed=17)
        st.prefill(dg["k"], dg["v"], dg["alpha"], dg["beta"])
        torch.cuda.synchronize()
        _check(cfg, st, before, dn, str(cfg))
    d2g, d2n = _inputs(_recipe(dc), cfg.n, cfg.dk, cfg.dv, 1, seed=18, t0=150)
    before = snapshot(st)
    o = st.step(d2g["q"][0], d2g["k"][0], d2g["v"][0], d2g["alpha"][0], d2g["beta"][0])
    rep = compare_step(ocfg_of(cfg, step=150), before,
                       tuple(d2n[x][0] for x in ("q", "k", "v", "alpha", "beta")), snapshot(st),
                       o.cpu().numpy())
    assert rep.ok, str(rep)


def test_prefill_from_zero_state_and_empty_prompt():
    cfg = lsq.LsqConfig(batch=1, heads=4, dk=64, dv=128, bits=8, group=64,
                        policy=lsq.POLICY_DYNAMIC, delta=0, decay=lsq.DECAY_SCALAR)
    st = _state(cfg, start_scale=0)
    before = snapshot(st)
    dg, dn = _inputs("la", cfg.n, cfg.dk, cfg.dv, 70)
    e = {k: v[:0] for k, v in dg.items()}
    st.prefill(e["k"], e["v"], e["alpha"], e["beta"])          # T = 0: nothing happens
    torch.cuda.synchronize()
    assert np.array_equal(snapshot(st).codes, before.codes) and st.step_index == 0
    st.prefill(dg["k"], dg["v"], dg["alpha"], dg["beta"])
    torch.cuda.synchronize()
    _check(cfg, st, before, dn, "from zero")


def test_prompt_split_at_chunk_boundaries_equals_one_call():
    cfg = lsq.LsqConfig(batch=1, heads=3, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_PERSISTENT, delta=0, decay=lsq.DECAY_DIAG)
    dg, dn = _inputs("gla", cfg.n, cfg.dk, cfg.dv, 200, seed=2)
    one = _state(cfg)
    before = snapshot(one)
    one.prefill(dg["k"], dg["v"], dg["alpha"], dg["beta"])
    split = _state(cfg)
    for a, b in ((0, 64), (64, 192), (192, 200)):
        split.prefill(*(dg[x][a:b].contiguous() for x in ("k", "v", "alpha", "beta")))
    torch.cuda.synchronize()
    s1, s2 = snapshot(one), snapshot(split)
    assert np.array_equal(s1.codes, s2.codes) and np.array_equal(s1.scales, s2.scales)
    assert split.step_index == 200
    _check(cfg, one, before, dn, "one call")


def test_decode_step_after_prefill():
    """The prefilled state is the decode step's state: a step taken after it
    meets the decode-step bar against the oracle."""
    cfg = lsq.LsqConfig(batch=2, heads=2, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_DYNAMIC, rounding=lsq.ROUND_BDR, delta=0,
                        decay=lsq.DECAY_DIAG)
    st = _state(cfg)
    before = snapshot(st)
    T = 100
    dg, dn = _inputs("gla", cfg.n, cfg.dk, cfg.dv, T + 1)
    st.prefill(*(dg[x][:T].contiguous() for x in ("k", "v", "alpha", "beta")))
    torch.cuda.synchronize()
    _check(cfg, st, before, {x: dn[x][:T] for x in dn}, "prefill")
    pre = snapshot(st)
    o = st.step(*(dg[x][T] for x in ("q", "k", "v", "alpha", "beta")))
    rep = compare_step(ocfg_of(cfg, step=T), pre,
                       tuple(dn[x][T] for x in ("q", "k", "v", "alpha", "beta")), snapshot(st),
                       o.cpu().numpy())
    assert rep.ok, str(rep)


def test_prefill_full_size_sampled_heads():
    """The timed workload's launch (batch 64 x 16 heads, 4096 tokens, INT4 g32
    dynamic, diagonal decay); the oracle follows four sampled heads."""
    wl = PREFILL_WORKLOADS["prefill-gla"]
    cfg = lsq.LsqConfig(**wl.config())
    st = lsq.LsqState(cfg, device=DEV).zero()
    n = cfg.n
    d = gen_steps(wl.recipe, n, cfg.dk, cfg.dv, [0], 0, wl.tokens, device=DEV)
    d = {k: d[k] for k in ("k", "v", "alpha", "beta")}
    st.prefill(d["k"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    heads = [0, 1, n // 2 + 7, n - 1]
    idx = torch.tensor(heads, device=DEV)
    sub = {k: v.index_select(1, idx).cpu().numpy() for k, v in d.items()}
    ocfg = oracle.OracleConfig(batch=1, heads=len(heads), dk=cfg.dk, dv=cfg.dv, bits=cfg.bits,
                               group=cfg.group, policy=cfg.policy, rounding=lsq.ROUND_RNE,
                               delta=0, decay=cfg.decay)
    want = oracle.zero_state(ocfg)
    oracle.prefill(ocfg, want, sub["k"], sub["v"], sub["alpha"], sub["beta"], chunk=64)
    got = snapshot(st, heads=heads)
    assert np.array_equal(got.codes, want.codes)
    assert np.array_equal(got.scales, want.scales)
    assert st.step_index == wl.tokens
