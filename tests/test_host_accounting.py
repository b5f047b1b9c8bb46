"""Byte and operation accounting of the benchmark (host logic, no GPU).

The roofline figures divide these counts by measured times, so each is pinned
here to a hand count for one configuration."""
import quantized_recurrent_state_amd as lsq
from quantized_recurrent_state_amd import runner
from quantized_recurrent_state_amd.inputs import PREFILL_WORKLOADS


def test_decode_step_bytes_int4_persistent_scalar():
    cfg = lsq.LsqConfig(batch=2, heads=3, dk=128, dv=128, bits=4, group=32,
                        policy=lsq.POLICY_PERSISTENT, delta=1)
    # per head: codes 128*64 B read + written, scales 128*4*4 B read only,
    # q, k (128 f32 each), v (128), alpha, beta (1 each) read, o (128) written
    per_head = 2 * 128 * 64 + 128 * 4 * 4 + 4 * (128 + 128 + 128 + 1 + 1) + 4 * 128
    assert runner.algorithmic_bytes(cfg) == 6 * per_head


def test_decode_step_bytes_yoked_diag_with_reference_output():
    cfg = lsq.LsqConfig(batch=1, heads=1, dk=64, dv=32, bits=8, group=64,
                        policy=lsq.POLICY_YOKED, decay=lsq.DECAY_DIAG)
    per_head = (2 * 32 * 64 + 2 * 32 * 1 * 4 + 2 * 4 * 32 * 64
                + 4 * (64 + 64 + 32 + 64 + 1) + 2 * 4 * 32)
    assert runner.algorithmic_bytes(cfg, with_o_ref=True) == per_head


def test_prefill_bytes_and_ops_of_the_timed_workload():
    wl = PREFILL_WORKLOADS["prefill-gla"]
    cfg = lsq.LsqConfig(**wl.config())
    assert (cfg.n, wl.tokens, cfg.dk, cfg.dv) == (1024, 4096, 128, 128)
    # per head: k, v, diagonal alpha (128 f32 each) and beta per token; codes
    # 128*64 B and scales 128*4 f32, each read and written (dynamic policy)
    per_head = 4 * 4096 * (128 + 128 + 128 + 1) + 2 * 128 * 64 + 2 * 128 * 4 * 4
    assert runner.prefill_algorithmic_bytes(cfg, wl.tokens) == 1024 * per_head == 6480199680
    assert runner.prefill_int8_ops(cfg, wl.tokens) == 2 * 1024 * 4096 * 128 * 128


def test_prefill_bytes_scalar_decay_persistent():
    cfg = lsq.LsqConfig(batch=1, heads=2, dk=64, dv=128, bits=8, group=32,
                        policy=lsq.POLICY_PERSISTENT)
    per_head = 4 * 100 * (64 + 128 + 1 + 1) + 2 * 128 * 64 + 128 * 2 * 4
    assert runner.prefill_algorithmic_bytes(cfg, 100) == 2 * per_head


def test_valu_issue_prices_the_hot_loop_at_the_probe_rates():
    """bench.valu_issue: one row-iteration's instructions, each at its probe
    rate (unlisted kinds at the med3 rate), times the rows, plus the set-up at
    the med3 rate; a hand count for a two-kind histogram."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    rec = {"instr_per_launch": 3.0e9, "waves_per_launch": 10, "row_iterations_per_wave": 4,
           "hot_loop_per_row_iteration": {"fma": 60, "other": 10}, "setup_per_wave": 20}
    ceiling = {"valu": {"fma": {"wave_instr_per_s": 1.0e6}, "med3": {"wave_instr_per_s": 0.5e6},
                        "fmac": {"wave_instr_per_s": 2.0e6}}}
    got = bench.valu_issue(rec, ceiling, launch_ms=2.0, nbytes=8_000_000)
    floor = 40 * (60 / 1.0e6 + 10 / 0.5e6) + 10 * 20 / 0.5e6      # seconds: 0.0032 + 0.0004
    assert abs(got["priced_floor_us"] - floor * 1e6) < 0.05
    assert abs(got["frac_of_priced_floor"] - floor / 2.0e-3) < 1e-4
    assert abs(got["achieved_wave_instr_per_s"] - 3.0e9 / 2.0e-3) < 1e7
    assert abs(got["hbm_frac_at_floor"] - 8_000_000 / floor / 8.0e12) < 1e-4
    assert bench.valu_issue(rec, None, 2.0, 1) is None
    assert bench.valu_issue(None, ceiling, 2.0, 1) is None
