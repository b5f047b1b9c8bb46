"""ctypes binding of liblsq.so (include/lsq.h).  Argument marshalling only.

Loading fails loudly when the library has not been built; there is no
fallback of any kind: every step of the decode path runs in the HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsq.so")
INCLUDE = os.path.join(os.path.dirname(_PKG), "include")
HEADER = os.path.join(INCLUDE, "lsq.h")

LSQ_OK = 0
STATUS_NAMES = {0: "LSQ_OK", 1: "LSQ_ERR_INVALID_ARG", 2: "LSQ_ERR_UNSUPPORTED",
                3: "LSQ_ERR_BUFFER_TOO_SMALL", 4: "LSQ_ERR_NOT_CALIBRATED", 5: "LSQ_ERR_HIP"}


class lsq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "dk", "dv", "bits", "group", "policy", "rounding", "delta",
                 "decay", "lrb_rank", "scale_fmt")]


class lsq_buffers(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("codes_bytes", ctypes.c_size_t),
                ("scales", ctypes.c_void_p), ("scales_bytes", ctypes.c_size_t),
                ("ref", ctypes.c_void_p), ("ref_bytes", ctypes.c_size_t),
                ("f32", ctypes.c_void_p), ("f32_bytes", ctypes.c_size_t),
                ("lrb", ctypes.c_void_p), ("lrb_bytes", ctypes.c_size_t)]


class LsqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


_lib = None


def load() -> ctypes.CDLL:
    """Load liblsq.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    cfgp = ctypes.POINTER(lsq_config)
    sig = {
        "lsq_state_sizes": [cfgp, ctypes.POINTER(S), ctypes.POINTER(S), ctypes.POINTER(S),
                            ctypes.POINTER(S), ctypes.POINTER(S)],
        "lsq_state_alloc": [cfgp, ctypes.POINTER(lsq_buffers), ctypes.POINTER(P)],
        "lsq_state_free": [P],
        "lsq_state_config": [P, cfgp],
        "lsq_state_zero": [P, P],
        "lsq_state_calibrate": [P, P, P],
        "lsq_state_dequantize": [P, P, P],
        "lsq_state_set_calibrated": [P, ctypes.c_int32],
        "lsq_state_step_index": [P, ctypes.POINTER(ctypes.c_int64)],
        "lsq_state_set_step_index": [P, ctypes.c_int64],
        "lsq_decode_step": [P, P, P, P, P, P, P, P, P],
        "lsq_decode_run": [P, ctypes.c_int32, P, P, P, P, P, P, P, P],
        "lsq_prefill": [P, ctypes.c_int32, P, P, P, P, P],
        "lsq_status_string": [ctypes.c_int],
        "lsq_last_error": [],
        "lsq_version": [],
        "lsq_probe_stream": [ctypes.c_int32, P, P, S, ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int32, P],
        "lsq_probe_span": [P, P, S, ctypes.c_int32, ctypes.c_int32, P],
        "lsq_probe_valu": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.lsq_state_free.restype = None
    L.lsq_status_string.restype = ctypes.c_char_p
    L.lsq_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != LSQ_OK:
        detail = load().lsq_last_error().decode()
        raise LsqError(status, where, detail)


def header_functions(paths: list[str] | None = None) -> list[str]:
    """Names of the functions the headers under include/ declare."""
    import glob
    names = set()
    for path in paths or sorted(glob.glob(os.path.join(INCLUDE, "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(lsq_[a-z_0-9]+)\s*\(", text))
    return sorted(names)
