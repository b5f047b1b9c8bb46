"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library loads, exports every function include/lsq.h declares, sizes the
state buffers as the packed layout defines, and rejects bad arguments with the
documented status before touching the device.  The device pointers used here
are never dereferenced: every call below fails validation (or is a no-op)
before any launch.
"""
import ctypes

import pytest

import quantized_recurrent_state_amd as lsq
from quantized_recurrent_state_amd import _lib

FAKE = 0x7F0000000000          # a 16-byte aligned address that is never touched


def test_every_declared_symbol_is_exported():
    L = _lib.load()
    names = _lib.header_functions()
    assert {"lsq_state_alloc", "lsq_decode_step", "lsq_decode_run"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert lsq.lsq_version() >= 100


@pytest.mark.parametrize("cfg,want", [
    # INT4 g32 128x128: 64 B codes + 4 scales per row
    (lsq.LsqConfig(2, 3, 128, 128, 4, 32, lsq.POLICY_PERSISTENT), (6 * 128 * 64, 6 * 128 * 16, 0, 0, 0)),
    # INT8 g64 Dv 64: 128 B codes + 2 scales per row
    (lsq.LsqConfig(1, 5, 128, 64, 8, 64, lsq.POLICY_DYNAMIC), (5 * 64 * 128, 5 * 64 * 8, 0, 0, 0)),
    # yoked adds the fp32 reference
    (lsq.LsqConfig(1, 1, 64, 64, 4, 32, lsq.POLICY_YOKED), (64 * 32, 64 * 8, 64 * 64 * 4, 0, 0)),
    # fp32 state
    (lsq.LsqConfig(1, 2, 64, 32, 32, 1, lsq.POLICY_NONE), (0, 0, 0, 2 * 32 * 64 * 4, 0)),
    # 16-bit scales: 2 bytes per group
    (lsq.LsqConfig(2, 3, 128, 128, 4, 32, lsq.POLICY_PERSISTENT, scale_fmt=lsq.SCALE_BF16),
     (6 * 128 * 64, 6 * 128 * 4 * 2, 0, 0, 0)),
    (lsq.LsqConfig(1, 1, 64, 64, 8, 16, lsq.POLICY_YOKED, scale_fmt=lsq.SCALE_F16),
     (64 * 64, 64 * 4 * 2, 64 * 64 * 4, 0, 0)),
    # one fp32 scale per head
    (lsq.LsqConfig(2, 3, 128, 128, 4, 0, lsq.POLICY_DYNAMIC), (6 * 128 * 64, 6 * 4, 0, 0, 0)),
    # bypass: a [n][r][Dv] + b [n][2][r][Dk] fp32
    (lsq.LsqConfig(1, 2, 128, 64, 4, 32, lsq.POLICY_PERSISTENT, lrb_rank=4),
     (2 * 64 * 64, 2 * 64 * 16, 0, 0, 2 * 4 * (64 + 2 * 128) * 4)),
])
def test_state_sizes(cfg, want):
    assert lsq.lsq_state_sizes(cfg) == want


BAD = [
    (dict(bits=5), 1), (dict(bits=32, policy=lsq.POLICY_DYNAMIC), 1),
    (dict(policy=lsq.POLICY_NONE), 1), (dict(group=48), 1),
    (dict(delta=2), 1), (dict(decay=3), 1), (dict(rounding=7), 1), (dict(batch=-1), 1),
    (dict(dk=96, group=32), 2), (dict(group=8), 2), (dict(bits=8, group=8), 2),
    (dict(group=24), 1), (dict(lrb_rank=9), 1), (dict(lrb_rank=-1), 1),
    (dict(lrb_rank=2, policy=lsq.POLICY_YOKED), 2), (dict(lrb_rank=2, group=16), 2),
    (dict(dk=256, group=32), 2),
    (dict(scale_fmt=3), 1), (dict(scale_fmt=-1), 1),
    (dict(rounding=5), 1), (dict(rounding=3, policy=lsq.POLICY_DYNAMIC), 1),
    (dict(group=-1), 1), (dict(group=0, policy=lsq.POLICY_YOKED), 1),
    (dict(group=0, rounding=2), 1), (dict(group=0, scale_fmt=2), 2),
    (dict(group=0, lrb_rank=2), 2), (dict(group=0, dv=1025), 2),
    (dict(rounding=4, policy=lsq.POLICY_YOKED), 1),
    (dict(rounding=4, policy=lsq.POLICY_PERSISTENT, group=16), 2),
    (dict(rounding=3, policy=lsq.POLICY_PERSISTENT, scale_fmt=2), 2),
    (dict(bits=32, group=1, policy=lsq.POLICY_NONE, scale_fmt=1), 1),
    (dict(lrb_rank=2, scale_fmt=2), 2),
]


@pytest.mark.parametrize("change,status", BAD)
def test_invalid_configs_are_rejected(change, status):
    base = dict(batch=1, heads=1, dk=128, dv=128, bits=4, group=32,
                policy=lsq.POLICY_PERSISTENT, rounding=0, delta=0, decay=0)
    base.update(change)
    cfg = lsq.LsqConfig(**base)
    with pytest.raises(lsq.LsqError) as e:
        lsq.lsq_state_sizes(cfg)
    assert e.value.status == status
    assert _lib.load().lsq_last_error().decode() != ""


def _alloc(cfg, codes=FAKE, cb=None, scales=FAKE, sb=None):
    L = _lib.load()
    need = lsq.lsq_state_sizes(cfg)
    bufs = _lib.lsq_buffers(codes, need[0] if cb is None else cb, scales,
                            need[1] if sb is None else sb, None, 0, None, 0, None, 0)
    h = ctypes.c_void_p()
    st = L.lsq_state_alloc(ctypes.byref(cfg.c()), ctypes.byref(bufs), ctypes.byref(h))
    return st, h.value


def test_alloc_checks_buffers():
    cfg = lsq.LsqConfig(1, 2, 128, 16, 4, 32, lsq.POLICY_PERSISTENT)
    assert _alloc(cfg, codes=None)[0] == 1
    assert _alloc(cfg, codes=FAKE + 8)[0] == 1                 # misaligned
    assert _alloc(cfg, cb=100)[0] == 3                         # too small
    st, h = _alloc(cfg)
    assert st == 0 and h
    out = _lib.lsq_config()
    assert _lib.load().lsq_state_config(h, ctypes.byref(out)) == 0 and out.dk == 128
    lsq.lsq_state_free(h)
    lsq.lsq_state_free(None)                                   # no-op


def test_step_argument_checks_before_launch():
    L = _lib.load()
    cfg = lsq.LsqConfig(1, 2, 128, 16, 4, 32, lsq.POLICY_PERSISTENT)
    st, h = _alloc(cfg)
    assert st == 0
    ptrs = [FAKE] * 6
    # persistent policy without calibration
    assert L.lsq_decode_step(h, *ptrs, None, None) == 4
    assert L.lsq_decode_run(h, 3, *ptrs, None, None) == 4
    assert L.lsq_state_set_calibrated(h, 1) == 0
    # null and misaligned inputs
    assert L.lsq_decode_step(h, None, *ptrs[1:], None, None) == 1
    assert L.lsq_decode_step(h, FAKE + 4, *ptrs[1:], None, None) == 1
    assert L.lsq_decode_run(h, -1, *ptrs, None, None) == 1
    assert L.lsq_decode_run(h, 0, *ptrs, None, None) == 0       # empty horizon
    assert L.lsq_decode_step(None, *ptrs, None, None) == 1
    lsq.lsq_state_free(h)


def test_empty_batch_calls_are_noops():
    L = _lib.load()
    cfg = lsq.LsqConfig(0, 4, 128, 128, 4, 32, lsq.POLICY_DYNAMIC)
    st, h = _alloc(cfg, codes=None, scales=None)
    assert st == 0
    assert L.lsq_decode_step(h, None, None, None, None, None, None, None, None) == 0
    assert L.lsq_state_calibrate(h, None, None) == 0
    assert L.lsq_state_dequantize(h, None, None) == 0
    lsq.lsq_state_free(h)


def test_dequantize_argument_checks_before_launch():
    L = _lib.load()
    cfg = lsq.LsqConfig(1, 2, 128, 16, 4, 32, lsq.POLICY_DYNAMIC)
    st, h = _alloc(cfg)
    assert st == 0
    assert L.lsq_state_dequantize(h, None, None) == 1           # null S
    assert L.lsq_state_dequantize(h, FAKE + 4, None) == 1       # misaligned S
    assert L.lsq_state_dequantize(None, FAKE, None) == 1        # null handle
    lsq.lsq_state_free(h)


def test_status_strings():
    for s in range(6):
        assert lsq.lsq_status_string(s).startswith(_lib.STATUS_NAMES[s])


def test_step_index_is_host_state():
    L = _lib.load()
    cfg = lsq.LsqConfig(1, 2, 128, 16, 4, 32, lsq.POLICY_DYNAMIC, lsq.ROUND_DITHER)
    st, h = _alloc(cfg)
    assert st == 0
    assert lsq.lsq_state_step_index(h) == 0
    lsq.lsq_state_set_step_index(h, 5)
    assert lsq.lsq_state_step_index(h) == 5
    with pytest.raises(lsq.LsqError) as e:
        lsq.lsq_state_set_step_index(h, -1)
    assert e.value.status == 1
    lsq.lsq_state_free(h)
    # an empty batch still advances the sequence position (no device work)
    cfg0 = lsq.LsqConfig(0, 4, 128, 128, 4, 32, lsq.POLICY_DYNAMIC, lsq.ROUND_DITHER)
    st, h = _alloc(cfg0, codes=None, scales=None)
    assert L.lsq_decode_step(h, None, None, None, None, None, None, None, None) == 0
    assert L.lsq_decode_run(h, 3, None, None, None, None, None, None, None, None) == 0
    assert lsq.lsq_state_step_index(h) == 4
    lsq.lsq_state_free(h)


def _alloc_all(cfg):
    """A handle whose every needed buffer is the untouched FAKE address."""
    L = _lib.load()
    need = lsq.lsq_state_sizes(cfg)
    p = [FAKE if n else None for n in need]
    bufs = _lib.lsq_buffers(p[0], need[0], p[1], need[1], p[2], need[2], p[3], need[3],
                            p[4], need[4])
    h = ctypes.c_void_p()
    assert L.lsq_state_alloc(ctypes.byref(cfg.c()), ctypes.byref(bufs), ctypes.byref(h)) == 0
    return h.value


@pytest.mark.parametrize("change", [
    dict(delta=1), dict(policy=lsq.POLICY_YOKED), dict(bits=32, group=1, policy=lsq.POLICY_NONE),
    dict(dv=32), dict(dv=256), dict(lrb_rank=2),
])
def test_prefill_rejects_unsupported_handles(change):
    base = dict(batch=1, heads=2, dk=128, dv=128, bits=4, group=32, policy=lsq.POLICY_DYNAMIC)
    base.update(change)
    cfg = lsq.LsqConfig(**base)
    h = _alloc_all(cfg)
    st = _lib.load().lsq_prefill(h, 64, FAKE, FAKE, FAKE, FAKE, None)
    assert st == 2, _lib.load().lsq_last_error()
    lsq.lsq_state_free(h)


def test_prefill_argument_checks_before_launch():
    L = _lib.load()
    cfg = lsq.LsqConfig(1, 2, 128, 64, 8, 16, lsq.POLICY_PERSISTENT)
    h = _alloc_all(cfg)
    p = [FAKE] * 4
    assert L.lsq_prefill(h, 64, *p, None) == 4                 # persistent, not calibrated
    assert L.lsq_state_set_calibrated(h, 1) == 0
    assert L.lsq_prefill(h, -1, *p, None) == 1                 # negative T
    assert L.lsq_prefill(h, 64, None, *p[1:], None) == 1       # null input
    assert L.lsq_prefill(h, 64, FAKE + 2, *p[1:], None) == 1   # misaligned input
    assert L.lsq_prefill(None, 64, *p, None) == 1
    assert lsq.lsq_state_step_index(h) == 0
    assert L.lsq_prefill(h, 0, *p, None) == 0                  # no tokens: nothing to do
    lsq.lsq_state_free(h)
    # an empty batch only advances the sequence position
    cfg0 = lsq.LsqConfig(0, 4, 128, 128, 4, 32, lsq.POLICY_DYNAMIC)
    st, h = _alloc(cfg0, codes=None, scales=None)
    assert L.lsq_prefill(h, 100, None, None, None, None, None) == 0
    assert lsq.lsq_state_step_index(h) == 100
    lsq.lsq_state_free(h)


def test_probe_argument_checks_before_launch():
    L = _lib.load()
    assert L.lsq_probe_stream(3, FAKE, FAKE, 4096, 4, 0, 0, None) == 1        # kind
    assert L.lsq_probe_stream(2, FAKE, FAKE, 4100, 4, 0, 0, None) == 1        # size % 16
    assert L.lsq_probe_stream(2, FAKE, FAKE, 4096, 3, 0, 0, None) == 1        # loads per lane
    assert L.lsq_probe_stream(2, FAKE, FAKE, 4096, 4, 2, 0, None) == 1        # nontemporal flag
    assert L.lsq_probe_stream(2, FAKE, FAKE, 4096, 4, 0, -1, None) == 1       # workgroups
    assert L.lsq_probe_stream(0, None, FAKE, 4096, 4, 0, 0, None) == 1        # read needs src
    assert L.lsq_probe_stream(2, FAKE + 4, FAKE, 4096, 4, 0, 0, None) == 1    # misaligned
    assert L.lsq_probe_stream(1, None, None, 4096, 4, 0, 0, None) == 1        # write needs dst
    assert L.lsq_probe_stream(2, FAKE, FAKE, 0, 4, 0, 0, None) == 0           # empty: no-op
    assert L.lsq_probe_stream(1, None, FAKE, 0, 1, 1, 7, None) == 0


def test_probe_valu_argument_checks_before_launch():
    L = _lib.load()
    assert L.lsq_probe_valu(10, 1024, 8, FAKE, None) == 1     # form
    assert L.lsq_probe_valu(-1, 1024, 8, FAKE, None) == 1
    assert L.lsq_probe_valu(0, 0, 8, FAKE, None) == 1         # workgroups
    assert L.lsq_probe_valu(1, 1024, 0, FAKE, None) == 1      # iterations
    assert L.lsq_probe_valu(2, 1024, 8, None, None) == 1      # null out


def test_probe_span_argument_checks_before_launch():
    L = _lib.load()
    assert L.lsq_probe_span(FAKE, FAKE, 10240, 3, 1, None) == 1        # span
    assert L.lsq_probe_span(FAKE, FAKE, 10240, 10, 2, None) == 1       # nontemporal flag
    assert L.lsq_probe_span(FAKE, FAKE, 10000, 10, 1, None) == 1       # not a whole number of spans
    assert L.lsq_probe_span(None, FAKE, 10240, 10, 1, None) == 1       # null source
    assert L.lsq_probe_span(FAKE, FAKE + 8, 10240, 10, 1, None) == 1   # misaligned
    assert L.lsq_probe_span(FAKE, FAKE, 0, 10, 1, None) == 0           # empty: no-op
