"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: every replay must reproduce the eager steps bit for bit.

The library's launches allocate nothing and record no memset, so a caller can
capture them; each captured launch keeps its own inputs, step index (dither
position) and bypass slot.  The test runs the steps eagerly, restores the
state, captures the same steps, and replays the graph several times with
eager work (state restore copies, a synchronisation) between replays,
comparing codes, scales, reference state, bypass slots and outputs with the
eager run after every replay.
"""
import pytest
import torch

import quantized_recurrent_state_amd as lsq
from quantized_recurrent_state_amd.inputs import gen_steps

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    dict(bits=4, group=32, policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_BDR, delta=1, decay=0),
    dict(bits=8, group=64, policy=lsq.POLICY_DYNAMIC, rounding=lsq.ROUND_RNE, delta=0, decay=1),
    dict(bits=4, group=32, policy=lsq.POLICY_DYNAMIC, rounding=lsq.ROUND_DITHER, delta=1, decay=0),
    dict(bits=4, group=32, policy=lsq.POLICY_YOKED, rounding=lsq.ROUND_RNE, delta=1, decay=0),
    dict(bits=4, group=32, policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_BDR, delta=1, decay=1,
         lrb_rank=2),
    dict(bits=4, group=0, policy=lsq.POLICY_DYNAMIC, rounding=lsq.ROUND_BDR, delta=1, decay=0),
    dict(bits=4, group=16, policy=lsq.POLICY_DYNAMIC, rounding=lsq.ROUND_BDR, delta=1, decay=0,
         scale_fmt=lsq.SCALE_BF16),
    dict(bits=8, group=64, policy=lsq.POLICY_PERSISTENT, rounding=lsq.ROUND_BDR_B, delta=0, decay=0),
]


def _buffers(st):
    return [b for b in (st.codes, st.scales, st.ref, st.lrb) if b is not None]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_graph_replays_equal_eager_steps(case):
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=128, dv=72, **case)
    st = lsq.LsqState(cfg, device=DEV).zero()
    g0 = torch.Generator(device=DEV).manual_seed(5)
    if cfg.policy == lsq.POLICY_PERSISTENT:
        st.calibrate(torch.randn(cfg.n, cfg.dv, cfg.dk, device=DEV, generator=g0) * 0.3)
    else:
        st.calibrate(torch.randn(cfg.n, cfg.dv, cfg.dk, device=DEV, generator=g0) * 0.3)
    H = 5                                     # covers a bypass merge (rank 2)
    recipe = "gla" if cfg.decay else "gdn"
    d = {k: v.to(DEV) for k, v in gen_steps(recipe, cfg.n, cfg.dk, cfg.dv, [3], 0, H).items()}
    yoked = cfg.policy == lsq.POLICY_YOKED
    saved = [b.clone() for b in _buffers(st)]
    t0 = st.step_index

    def steps(o, o_ref, stream):
        for t in range(H):
            lsq.lsq_decode_step(st.handle, d["q"][t], d["k"][t], d["v"][t], d["alpha"][t],
                                d["beta"][t], o[t], o_ref[t] if yoked else None, stream)

    # eager reference
    o_e = torch.empty(H, cfg.n, cfg.dv, device=DEV)
    r_e = torch.empty(H, cfg.n, cfg.dv, device=DEV)
    steps(o_e, r_e, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [b.clone() for b in _buffers(st)]

    # capture the same steps from the same state
    for b, s0 in zip(_buffers(st), saved):
        b.copy_(s0)
    st.step_index = t0
    o_g = torch.zeros(H, cfg.n, cfg.dv, device=DEV)
    r_g = torch.zeros(H, cfg.n, cfg.dv, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(o_g, r_g, torch.cuda.current_stream())
    assert st.step_index == t0 + H
    for rep in range(3):
        for b, s0 in zip(_buffers(st), saved):    # eager work between replays
            b.copy_(s0)
        o_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for b, w in zip(_buffers(st), want):
            assert torch.equal(b, w), (rep, case)
        assert torch.equal(o_g, o_e), (rep, case)
        if yoked:
            assert torch.equal(r_g, r_e), (rep, case)
