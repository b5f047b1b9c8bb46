"""Low-bit recurrent-state decode step for MI355X: Python binding of liblsq.so.

The functions below carry the names of the C ABI in ``include/lsq.h`` and do
argument marshalling only; PyTorch provides device memory and streams.  Every
step of the decode path runs in the library's HIP kernels.  Importing this
package does not load the library; the first call does, and fails loudly if
it has not been built.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, asdict

from . import _lib
from ._lib import LsqError

POLICY_NONE, POLICY_DYNAMIC, POLICY_PERSISTENT, POLICY_YOKED = 0, 1, 2, 3
ROUND_RNE, ROUND_BDR, ROUND_DITHER = 0, 1, 2
ROUND_BDR_A, ROUND_BDR_B = 3, 4        # rejected directional readings (sensitivity flags)
DECAY_SCALAR, DECAY_DIAG = 0, 1
SCALE_F32, SCALE_F16, SCALE_BF16 = 0, 1, 2

__all__ = ["LsqConfig", "LsqState", "LsqError", "lsq_state_sizes", "lsq_state_alloc",
           "lsq_state_free", "lsq_state_zero", "lsq_state_calibrate", "lsq_state_dequantize", "lsq_state_set_calibrated",
           "lsq_state_step_index", "lsq_state_set_step_index",
           "lsq_decode_step", "lsq_decode_run", "lsq_prefill", "lsq_status_string", "lsq_version",
           "lsq_probe_stream", "lsq_probe_span",
           "lsq_probe_valu"]


@dataclass(frozen=True)
class LsqConfig:
    """Mirror of ``lsq_config``."""
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
    lrb_rank: int = 0       # Low-Rank Bypass slots (0: off)
    scale_fmt: int = SCALE_F32   # stored group-scale format

    @property
    def n(self) -> int:
        return self.batch * self.heads

    def c(self) -> _lib.lsq_config:
        return _lib.lsq_config(**asdict(self))


def _stream_ptr(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def lsq_state_sizes(cfg: LsqConfig) -> tuple[int, int, int, int, int]:
    """(codes, scales, ref, f32, lrb) byte sizes of the state buffers."""
    L = _lib.load()
    out = [ctypes.c_size_t(0) for _ in range(5)]
    _lib.check(L.lsq_state_sizes(ctypes.byref(cfg.c()), *map(ctypes.byref, out)),
               "lsq_state_sizes")
    return tuple(int(x.value) for x in out)


def lsq_state_alloc(cfg: LsqConfig, codes=None, scales=None, ref=None, f32=None,
                    lrb=None) -> int:
    """Bind caller-owned device tensors to a new handle (returns the handle)."""
    L = _lib.load()
    nb = lambda t: 0 if t is None else t.numel() * t.element_size()
    bufs = _lib.lsq_buffers(_ptr(codes), nb(codes), _ptr(scales), nb(scales), _ptr(ref), nb(ref),
                            _ptr(f32), nb(f32), _ptr(lrb), nb(lrb))
    h = ctypes.c_void_p()
    _lib.check(L.lsq_state_alloc(ctypes.byref(cfg.c()), ctypes.byref(bufs), ctypes.byref(h)),
               "lsq_state_alloc")
    return h.value


def lsq_state_free(handle: int) -> None:
    _lib.load().lsq_state_free(handle)


def lsq_state_zero(handle: int, stream=None) -> None:
    _lib.check(_lib.load().lsq_state_zero(handle, _stream_ptr(stream)), "lsq_state_zero")


def lsq_state_calibrate(handle: int, S, stream=None) -> None:
    _lib.check(_lib.load().lsq_state_calibrate(handle, _ptr(S), _stream_ptr(stream)),
               "lsq_state_calibrate")


def lsq_state_dequantize(handle: int, S, stream=None) -> None:
    _lib.check(_lib.load().lsq_state_dequantize(handle, _ptr(S), _stream_ptr(stream)),
               "lsq_state_dequantize")


def lsq_state_set_calibrated(handle: int, calibrated: bool = True) -> None:
    _lib.check(_lib.load().lsq_state_set_calibrated(handle, int(bool(calibrated))),
               "lsq_state_set_calibrated")


def lsq_state_step_index(handle: int) -> int:
    t = ctypes.c_int64(0)
    _lib.check(_lib.load().lsq_state_step_index(handle, ctypes.byref(t)), "lsq_state_step_index")
    return int(t.value)


def lsq_state_set_step_index(handle: int, t: int) -> None:
    _lib.check(_lib.load().lsq_state_set_step_index(handle, int(t)), "lsq_state_set_step_index")


def lsq_decode_step(handle: int, q, k, v, alpha, beta, o, o_ref=None, stream=None) -> None:
    _lib.check(_lib.load().lsq_decode_step(handle, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                           _ptr(beta), _ptr(o), _ptr(o_ref), _stream_ptr(stream)),
               "lsq_decode_step")


def lsq_decode_run(handle: int, H: int, q, k, v, alpha, beta, o, o_ref=None, stream=None) -> None:
    _lib.check(_lib.load().lsq_decode_run(handle, int(H), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                          _ptr(beta), _ptr(o), _ptr(o_ref), _stream_ptr(stream)),
               "lsq_decode_run")


def lsq_prefill(handle: int, T: int, k, v, alpha, beta, stream=None) -> None:
    _lib.check(_lib.load().lsq_prefill(handle, int(T), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _stream_ptr(stream)),
               "lsq_prefill")


def lsq_status_string(status: int) -> str:
    return _lib.load().lsq_status_string(int(status)).decode()


def lsq_version() -> int:
    return int(_lib.load().lsq_version())


PROBE_READ, PROBE_WRITE, PROBE_COPY = 0, 1, 2


def lsq_probe_stream(kind: int, src, dst, nbytes: int, loads_per_lane: int = 4,
                     nontemporal: int = 0, workgroups: int = 0, stream=None) -> None:
    """One streaming pass (include/lsq_probe.h) over device tensors src/dst."""
    _lib.check(_lib.load().lsq_probe_stream(kind, _ptr(src), _ptr(dst), nbytes, loads_per_lane,
                                            nontemporal, workgroups, _stream_ptr(stream)),
               "lsq_probe_stream")


def lsq_probe_span(src, dst, nbytes: int, span_kib: int = 10, nontemporal: int = 1,
                   stream=None) -> None:
    """Every wave walks its own span of src, rewriting it to dst (include/lsq_probe.h)."""
    _lib.check(_lib.load().lsq_probe_span(_ptr(src), _ptr(dst), nbytes, span_kib, nontemporal,
                                          _stream_ptr(stream)), "lsq_probe_span")


PROBE_VALU_FMA, PROBE_VALU_MED3, PROBE_VALU_MIXED = 0, 1, 2
PROBE_VALU_FMAC, PROBE_VALU_FMA_MIX, PROBE_VALU_LSHL_OR, PROBE_VALU_PERM = 3, 4, 5, 6
PROBE_VALU_XAD, PROBE_VALU_AND, PROBE_VALU_MUL = 7, 8, 9


def lsq_probe_valu(form: int, workgroups: int, iters: int, out, stream=None) -> None:
    """VALU issue probe (include/lsq_probe.h): workgroups * 4 * iters * 8 wave64
    instructions of one form; out is a device tensor of at least 4 bytes."""
    _lib.check(_lib.load().lsq_probe_valu(form, workgroups, iters, _ptr(out), _stream_ptr(stream)),
               "lsq_probe_valu")


class LsqState:
    """A handle plus the torch device buffers it binds (codes, scales, ref, f32)."""

    def __init__(self, cfg: LsqConfig, device="cuda"):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        _, _, n_ref, n_f32, n_lrb = lsq_state_sizes(cfg)
        n, dv, dk = cfg.n, cfg.dv, cfg.dk
        self.codes = self.scales = self.ref = self.f32 = self.lrb = None
        if cfg.bits != 32:
            self.codes = torch.empty((n, dv, dk * cfg.bits // 8), dtype=torch.uint8,
                                     device=self.device)
            sdt = {SCALE_F32: torch.float32, SCALE_F16: torch.float16,
                   SCALE_BF16: torch.bfloat16}[cfg.scale_fmt]
            sshape = (n, dv, dk // cfg.group) if cfg.group else (n, 1, 1)   # group 0: per head
            self.scales = torch.empty(sshape, dtype=sdt, device=self.device)
        if n_ref:
            self.ref = torch.empty((n, dv, dk), dtype=torch.float32, device=self.device)
        if cfg.bits == 32:
            self.f32 = torch.empty((n, dv, dk), dtype=torch.float32, device=self.device)
        if n_lrb:
            self.lrb = torch.empty(n_lrb // 4, dtype=torch.float32, device=self.device)
        self.handle = lsq_state_alloc(cfg, self.codes, self.scales, self.ref, self.f32, self.lrb)

    @property
    def lrb_a(self):
        """Bypass slots a: view [n, r, Dv] of the buffer (None without bypass)."""
        if self.lrb is None:
            return None
        c = self.cfg
        return self.lrb[: c.n * c.lrb_rank * c.dv].view(c.n, c.lrb_rank, c.dv)

    @property
    def lrb_b(self):
        """Bypass slots b: view [n, 2, r, Dk] (copy 1 used by diagonal decay)."""
        if self.lrb is None:
            return None
        c = self.cfg
        return self.lrb[c.n * c.lrb_rank * c.dv:].view(c.n, 2, c.lrb_rank, c.dk)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                lsq_state_free(h)
            except Exception:
                pass
            self.handle = None

    def zero(self, stream=None):
        lsq_state_zero(self.handle, stream)
        return self

    def calibrate(self, S, stream=None):
        _check_tensor("S", S, (self.cfg.n, self.cfg.dv, self.cfg.dk))
        lsq_state_calibrate(self.handle, S, stream)
        return self

    def dequantize(self, out=None, stream=None):
        """fl(C s) of every element as an fp32 tensor [n, dv, dk] (the stored state)."""
        import torch
        if out is None:
            out = torch.empty((self.cfg.n, self.cfg.dv, self.cfg.dk), device=self.device,
                              dtype=torch.float32)
        _check_tensor("out", out, (self.cfg.n, self.cfg.dv, self.cfg.dk))
        lsq_state_dequantize(self.handle, out, stream)
        return out

    def set_calibrated(self, calibrated=True):
        lsq_state_set_calibrated(self.handle, calibrated)
        return self

    @property
    def step_index(self) -> int:
        """Sequence position of the next step (dithered rounding)."""
        return lsq_state_step_index(self.handle)

    @step_index.setter
    def step_index(self, t: int) -> None:
        lsq_state_set_step_index(self.handle, t)

    def _out(self, o, lead):
        import torch
        if o is None:
            o = torch.empty(lead + (self.cfg.n, self.cfg.dv), device=self.device,
                            dtype=torch.float32)
        return o

    def _check_inputs(self, q, k, v, alpha, beta, lead=()):
        c = self.cfg
        _check_tensor("q", q, lead + (c.n, c.dk))
        _check_tensor("k", k, lead + (c.n, c.dk))
        _check_tensor("v", v, lead + (c.n, c.dv))
        _check_tensor("alpha", alpha, lead + ((c.n, c.dk) if c.decay == DECAY_DIAG else (c.n,)))
        _check_tensor("beta", beta, lead + (c.n,))

    def step(self, q, k, v, alpha, beta, o=None, o_ref=None, stream=None):
        """One decode step; returns o (and o_ref for the yoked policy)."""
        self._check_inputs(q, k, v, alpha, beta)
        o = self._out(o, ())
        if self.cfg.policy == POLICY_YOKED and o_ref is None:
            o_ref = self._out(None, ())
        lsq_decode_step(self.handle, q, k, v, alpha, beta, o, o_ref, stream)
        return (o, o_ref) if self.cfg.policy == POLICY_YOKED else o

    def run(self, q, k, v, alpha, beta, o=None, o_ref=None, stream=None):
        """H decode steps (inputs with a leading [H] axis); returns o [H, n, Dv]."""
        H = int(q.shape[0])
        self._check_inputs(q, k, v, alpha, beta, lead=(H,))
        o = self._out(o, (H,))
        if self.cfg.policy == POLICY_YOKED and o_ref is None:
            o_ref = self._out(None, (H,))
        lsq_decode_run(self.handle, H, q, k, v, alpha, beta, o, o_ref, stream)
        return (o, o_ref) if self.cfg.policy == POLICY_YOKED else o

    def prefill(self, k, v, alpha, beta, stream=None):
        """Chunkwise prefill over T tokens (inputs with a leading [T] axis, no q)."""
        c = self.cfg
        T = int(k.shape[0])
        _check_tensor("k", k, (T, c.n, c.dk))
        _check_tensor("v", v, (T, c.n, c.dv))
        _check_tensor("alpha", alpha, (T,) + ((c.n, c.dk) if c.decay == DECAY_DIAG else (c.n,)))
        _check_tensor("beta", beta, (T, c.n))
        lsq_prefill(self.handle, T, k, v, alpha, beta, stream)
        return self


def _check_tensor(name, t, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
