"""CPU oracle for the low-bit recurrent-state decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``quantized_recurrent_state_amd``) and imports nothing
from it; the two meet only through inputs produced by the seeded generators.

The arithmetic lives in ``lsq_oracle.c`` (plain scalar C, see its header for
the passages of the pages each step follows).  This module builds it with gcc
when needed and marshals numpy arrays to it.

Parity pins (tests/test_oracle_*.py) tie every function here to something
other than itself: closed forms of Eq. (1) (LinQuant summary, Theoretical
Foundation), exact-rational brute force of the rounding rules, and invariants
of the quantiser.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field, asdict

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsq_oracle.c")
_HDR = os.path.join(_HERE, "lsq_oracle.h")
_LIB = os.path.join(_HERE, "liblsq_oracle.so")

POLICY_NONE, POLICY_DYNAMIC, POLICY_PERSISTENT, POLICY_YOKED = 0, 1, 2, 3
ROUND_RNE, ROUND_BDR, ROUND_DITHER = 0, 1, 2
ROUND_BDR_A, ROUND_BDR_B = 3, 4        # rejected directional readings (persistent scale only)
DECAY_SCALAR, DECAY_DIAG = 0, 1
SCALE_F32, SCALE_F16, SCALE_BF16 = 0, 1, 2

GCC_FLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
             "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm", "-pthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "dk", "dv", "bits", "group", "policy", "rounding", "delta",
                 "decay", "lrb_rank", "scale_fmt")] + [("step", ctypes.c_int64)]


class _Stats(ctypes.Structure):
    _fields_ = [("clamped", ctypes.c_int64), ("bdr_fired", ctypes.c_int64)]


_lib = None
_lib_lock = threading.Lock()


def lib():
    global _lib
    with _lib_lock:
        if _lib is None:
            _lib = _load(build())
        return _lib


def _load(path: str):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(_Config)
    L.lsqo_check_config.argtypes = [cfgp]
    L.lsqo_step.argtypes = [cfgp, P, P, P, P, P, P, P, P, P, P, P, ctypes.POINTER(_Stats)]
    L.lsqo_step_trace.argtypes = [cfgp, P, P, P, P, P, P, P, P, P, P, P,
                                  ctypes.POINTER(_Stats), P, P]
    L.lsqo_run.argtypes = [cfgp, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P, P,
                           ctypes.c_int32]
    L.lsqo_calibrate.argtypes = [cfgp, P, P, P, P, P]
    L.lsqo_step_lrb.argtypes = [cfgp, P, P, P, P, P, P, P, P, P, P,
                                ctypes.POINTER(_Stats), P, P]
    L.lsqo_prefill.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P]
    L.lsqo_dequantize.argtypes = [cfgp, P, P, P]
    L.lsqo_pack.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P, P]
    L.lsqo_unpack.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P, P]
    for f in (L.lsqo_check_config, L.lsqo_step, L.lsqo_step_trace, L.lsqo_run, L.lsqo_calibrate,
              L.lsqo_step_lrb, L.lsqo_prefill,
              L.lsqo_dequantize, L.lsqo_pack, L.lsqo_unpack):
        f.restype = ctypes.c_int
    L.lsqo_scale_as_stored.argtypes = [ctypes.c_float, ctypes.c_int32]
    L.lsqo_scale_as_stored.restype = ctypes.c_float
    return L


@contextlib.contextmanager
def planted(edits):
    """TEST SUPPORT: inside the block every function of this module runs an
    oracle built from lsq_oracle.c with the given (old, new) source edits
    applied: a planted mistake, compiled on the CPU into a temporary
    directory, to show that a pin catches it.  Each old text must occur in the
    source exactly once."""
    global _lib
    import tempfile
    text = open(_SRC).read()
    for old, new in edits:
        if text.count(old) != 1:
            raise ValueError(f"planted edit does not match exactly once: {old!r}")
        text = text.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "lsq_oracle.c")
        with open(src, "w") as f:
            f.write(text)
        out = os.path.join(d, "liblsq_oracle_planted.so")
        subprocess.run(["gcc", *GCC_FLAGS, f"-I{_HERE}", "-o", out, src, "-lm", "-pthread"],
                       check=True)
        keep = lib()
        with _lib_lock:
            _lib = _load(out)
        try:
            yield
        finally:
            with _lib_lock:
                _lib = keep


@dataclass(frozen=True)
class OracleConfig:
    """Shape, format and method flags of one decode-step configuration."""
    batch: int
    heads: int
    dk: int
    dv: int
    bits: int = 4
    group: int = 32
    policy: int = POLICY_PERSISTENT
    rounding: int = ROUND_RNE
    delta: int = 0
    decay: int = DECAY_SCALAR
    lrb_rank: int = 0      # Low-Rank Bypass slots (0: off)
    scale_fmt: int = 0     # stored scale format: 0 fp32, 1 binary16, 2 bfloat16
    step: int = 0          # sequence position of the (first) step: dithered rounding, bypass slot

    @property
    def n(self) -> int:
        return self.batch * self.heads

    @property
    def qmax(self) -> int:
        return (1 << (self.bits - 1)) - 1

    @property
    def ngroups(self) -> int:
        return self.dk // self.group if self.group else 1

    def c(self) -> _Config:
        return _Config(**asdict(self))

    def replace(self, **kw) -> "OracleConfig":
        d = asdict(self)
        d.update(kw)
        return OracleConfig(**d)


@dataclass
class OracleState:
    """Unpacked host state: signed codes, group scales, fp32 reference, fp32 state."""
    codes: np.ndarray | None = None   # int8  [n, Dv, Dk]
    scales: np.ndarray | None = None  # f32   [n, Dv, Dk/g]
    ref: np.ndarray | None = None     # f32   [n, Dv, Dk]  (yoked policy)
    f32: np.ndarray | None = None     # f32   [n, Dv, Dk]  (bits == 32)
    lrb_a: np.ndarray | None = None   # f32   [n, r, Dv]   (Low-Rank Bypass)
    lrb_b: np.ndarray | None = None   # f32   [n, r, Dk]

    def copy(self) -> "OracleState":
        return OracleState(*(None if a is None else a.copy()
                             for a in (self.codes, self.scales, self.ref, self.f32, self.lrb_a,
                                       self.lrb_b)))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def zero_state(cfg: OracleConfig) -> OracleState:
    """S_0 = 0 in every buffer the configuration uses."""
    n = cfg.n
    if cfg.bits == 32:
        return OracleState(f32=np.zeros((n, cfg.dv, cfg.dk), np.float32))
    st = OracleState(codes=np.zeros((n, cfg.dv, cfg.dk), np.int8),
                     scales=np.zeros((n, cfg.dv, cfg.ngroups) if cfg.group else (n, 1, 1),
                                     np.float32))
    if cfg.policy == POLICY_YOKED:
        st.ref = np.zeros((n, cfg.dv, cfg.dk), np.float32)
    if cfg.lrb_rank > 0:
        st.lrb_a = np.zeros((n, cfg.lrb_rank, cfg.dv), np.float32)
        st.lrb_b = np.zeros((n, cfg.lrb_rank, cfg.dk), np.float32)
    return st


def _check(cfg: OracleConfig):
    if lib().lsqo_check_config(ctypes.byref(cfg.c())) != 0:
        raise ValueError(f"oracle: invalid configuration {cfg}")


def _inputs(cfg, q, k, v, alpha, beta, lead=()):
    n = cfg.n
    q, k, v, alpha, beta = map(_f32, (q, k, v, alpha, beta))
    ashape = lead + ((n, cfg.dk) if cfg.decay == DECAY_DIAG else (n,))
    for name, a, shp in (("q", q, lead + (n, cfg.dk)), ("k", k, lead + (n, cfg.dk)),
                         ("v", v, lead + (n, cfg.dv)), ("alpha", alpha, ashape),
                         ("beta", beta, lead + (n,))):
        if a.shape != shp:
            raise ValueError(f"oracle: {name} has shape {a.shape}, expected {shp}")
    return q, k, v, alpha, beta


def step(cfg: OracleConfig, st: OracleState, q, k, v, alpha, beta, stats: dict | None = None,
         trace: dict | None = None):
    """One decode step of every head, in place on ``st``.

    Returns (o, o_ref); o_ref is None unless the policy is yoked.  With a
    ``trace`` dict (quantised states only), trace["y"] and trace["yp"] receive
    the exact pre-rounding values S_t*inv and S'*inv in code units (dithered
    rounding: trace["yp"] holds the dither offset u instead of S'*inv).
    """
    _check(cfg)
    q, k, v, alpha, beta = _inputs(cfg, q, k, v, alpha, beta)
    o = np.empty((cfg.n, cfg.dv), np.float32)
    o_ref = np.empty((cfg.n, cfg.dv), np.float32) if cfg.policy == POLICY_YOKED else None
    s = _Stats()
    y = yp = None
    if trace is not None and cfg.bits != 32:
        y = np.zeros((cfg.n, cfg.dv, cfg.dk), np.float64)
        yp = np.zeros((cfg.n, cfg.dv, cfg.dk), np.float64)
        trace["y"], trace["yp"] = y, yp
    if cfg.lrb_rank > 0:
        rc = lib().lsqo_step_lrb(ctypes.byref(cfg.c()), _p(st.codes), _p(st.scales), _p(st.lrb_a),
                                 _p(st.lrb_b), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(o),
                                 ctypes.byref(s), _p(y), _p(yp))
        if rc:
            raise RuntimeError("oracle bypass step failed")
        if stats is not None:
            stats["clamped"] = stats.get("clamped", 0) + s.clamped
            stats["bdr_fired"] = stats.get("bdr_fired", 0) + s.bdr_fired
        return o, None
    rc = lib().lsqo_step_trace(ctypes.byref(cfg.c()), _p(st.codes), _p(st.scales), _p(st.ref),
                               _p(st.f32), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(o),
                               _p(o_ref), ctypes.byref(s), _p(y), _p(yp))
    if rc:
        raise RuntimeError("oracle step failed")
    if stats is not None:
        stats["clamped"] = stats.get("clamped", 0) + s.clamped
        stats["bdr_fired"] = stats.get("bdr_fired", 0) + s.bdr_fired
    return o, o_ref


def run(cfg: OracleConfig, st: OracleState, q, k, v, alpha, beta, nthreads: int = 1):
    """H consecutive steps (inputs with a leading [H] axis); returns o [H, n, Dv]
    and o_ref (yoked policy) or None."""
    _check(cfg)
    H = int(np.shape(q)[0])
    q, k, v, alpha, beta = _inputs(cfg, q, k, v, alpha, beta, lead=(H,))
    o = np.empty((H, cfg.n, cfg.dv), np.float32)
    o_ref = np.empty((H, cfg.n, cfg.dv), np.float32) if cfg.policy == POLICY_YOKED else None
    rc = lib().lsqo_run(ctypes.byref(cfg.c()), H, _p(st.codes), _p(st.scales), _p(st.ref),
                        _p(st.f32), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(o), _p(o_ref),
                        int(nthreads))
    if rc:
        raise RuntimeError("oracle run failed")
    return o, o_ref


def prefill(cfg: OracleConfig, st: OracleState, k, v, alpha, beta, chunk: int = 64) -> None:
    """Chunkwise prefill of T tokens (inputs with a leading [T] axis) into the
    quantised state ``st``, in place (linear write, delta = 0)."""
    _check(cfg)
    T = int(np.shape(k)[0])
    n = cfg.n
    k, v, alpha, beta = map(_f32, (k, v, alpha, beta))
    ashape = (T, n, cfg.dk) if cfg.decay == DECAY_DIAG else (T, n)
    for name, a, shp in (("k", k, (T, n, cfg.dk)), ("v", v, (T, n, cfg.dv)),
                         ("alpha", alpha, ashape), ("beta", beta, (T, n))):
        if a.shape != shp:
            raise ValueError(f"oracle: {name} has shape {a.shape}, expected {shp}")
    rc = lib().lsqo_prefill(ctypes.byref(cfg.c()), T, int(chunk), _p(st.codes), _p(st.scales),
                            _p(k), _p(v), _p(alpha), _p(beta))
    if rc:
        raise RuntimeError("oracle prefill failed")


def scale_as_stored(s: float, fmt: int) -> float:
    """A group scale rounded to its stored format (SCALE_*), as an fp32 value."""
    return float(np.float32(lib().lsqo_scale_as_stored(float(s), int(fmt))))


def calibrate(cfg: OracleConfig, S) -> OracleState:
    """Quantise an fp32 state [n, Dv, Dk] (absmax group scales, RNE codes)."""
    _check(cfg)
    S = _f32(S)
    if S.shape != (cfg.n, cfg.dv, cfg.dk):
        raise ValueError("oracle: calibrate expects [n, Dv, Dk]")
    st = zero_state(cfg)
    rc = lib().lsqo_calibrate(ctypes.byref(cfg.c()), _p(S), _p(st.codes), _p(st.scales),
                              _p(st.ref), _p(st.f32))
    if rc:
        raise RuntimeError("oracle calibrate failed")
    return st


def dequantize(cfg: OracleConfig, st: OracleState) -> np.ndarray:
    """codes * scale as fp32 [n, Dv, Dk]."""
    out = np.empty((cfg.n, cfg.dv, cfg.dk), np.float32)
    rc = lib().lsqo_dequantize(ctypes.byref(cfg.c()), _p(st.codes), _p(st.scales), _p(out))
    if rc:
        raise RuntimeError("oracle dequantize failed")
    return out


def pack(codes, bits: int) -> np.ndarray:
    """Signed codes [..., Dk] -> packed bytes [..., Dk*bits/8] (layout in lsq_oracle.h)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    dk = codes.shape[-1]
    rows = codes.size // dk
    out = np.empty(codes.shape[:-1] + (dk * bits // 8,), np.uint8)
    if lib().lsqo_pack(bits, dk, rows, _p(codes), _p(out)):
        raise ValueError("oracle pack: unsupported bits/Dk")
    return out


def unpack(packed, bits: int, dk: int) -> np.ndarray:
    """Packed bytes [..., Dk*bits/8] -> signed codes [..., Dk]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    nb = dk * bits // 8
    if packed.shape[-1] != nb:
        raise ValueError("oracle unpack: last axis must hold Dk*bits/8 bytes")
    rows = packed.size // nb
    out = np.empty(packed.shape[:-1] + (dk,), np.int8)
    if lib().lsqo_unpack(bits, dk, rows, _p(packed), _p(out)):
        raise ValueError("oracle unpack: unsupported bits/Dk")
    return out


def fp32_warmup_then_calibrate(cfg: OracleConfig, q, k, v, alpha, beta, nthreads: int = 1):
    """Persistent-scale set-up: W fp32 steps from S_0 = 0 (inputs with a leading
    [W] axis), then freeze the group scales of S_W.  Returns (state, S_W)."""
    fcfg = cfg.replace(bits=32, policy=POLICY_NONE, rounding=ROUND_RNE)
    fst = zero_state(fcfg)
    run(fcfg, fst, q, k, v, alpha, beta, nthreads=nthreads)
    return calibrate(cfg, fst.f32), fst.f32
