"""ctypes declarations of the libelsaa C ABI (include/elsaa.h). Argument
marshalling only: every step of the operator runs in the library's kernels."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libelsaa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
STATUS_NAMES = {0: "ELSAA_OK", 1: "ELSAA_ERR_INVALID_ARG", 2: "ELSAA_ERR_UNSUPPORTED",
                3: "ELSAA_ERR_WORKSPACE", 4: "ELSAA_ERR_HIP"}
F32, BF16 = 0, 1
CALL_SELECT, CALL_SUMMARY, CALL_FWD, CALL_BWD, CALL_GATES_BWD, CALL_CHECK, CALL_TOPK = range(7)

SYMBOLS = ("elsaa_workspace_size", "elsaa_select", "elsaa_select_noalloc",
           "elsaa_lowrank_summary", "elsaa_fwd", "elsaa_bwd", "elsaa_fwd_fused", "elsaa_gates_fwd",
           "elsaa_gates_bwd", "elsaa_topk", "elsaa_check_orders", "elsaa_profile",
           "elsaa_profile_report", "elsaa_last_error")


class Params(ctypes.Structure):
    """elsaa_params."""
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("block", ctypes.c_int32), ("hash_bits", ctypes.c_int32),
                ("lr_tables", ctypes.c_int32), ("lr_bits", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("tau", ctypes.c_float), ("eps", ctypes.c_float),
                ("scale", ctypes.c_float), ("hash_rounds", ctypes.c_int32),
                ("extra_edges", ctypes.c_int32)]


class ElsaaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_vp = ctypes.c_void_p
_PP = ctypes.POINTER(Params)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_rank_approximation_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    L.elsaa_workspace_size.argtypes = [_PP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    L.elsaa_select.argtypes = [_PP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.elsaa_select_noalloc.argtypes = [_PP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.elsaa_lowrank_summary.argtypes = [_PP, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.elsaa_fwd.argtypes = [_PP] + [_vp] * 18 + [ctypes.c_size_t, _vp]
    L.elsaa_bwd.argtypes = [_PP] + [_vp] * 24 + [ctypes.c_size_t, _vp]
    L.elsaa_fwd_fused.argtypes = [_PP] + [_vp] * 20
    L.elsaa_gates_fwd.argtypes = [_PP] + [_vp] * 6
    L.elsaa_gates_bwd.argtypes = [_PP] + [_vp] * 10 + [ctypes.c_size_t, _vp]
    L.elsaa_topk.argtypes = [_PP, _vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_size_t, _vp]
    L.elsaa_check_orders.argtypes = [_PP] + [_vp] * 4 + [ctypes.c_size_t, _vp]
    L.elsaa_profile.argtypes = [ctypes.c_int32]
    L.elsaa_profile_report.argtypes = [ctypes.c_char_p, ctypes.c_size_t,
                                       ctypes.POINTER(ctypes.c_size_t)]
    L.elsaa_last_error.argtypes = []
    L.elsaa_last_error.restype = ctypes.c_char_p
    for s in SYMBOLS[:-1]:
        getattr(L, s).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int) -> None:
    if status != OK:
        raise ElsaaError(status, lib().elsaa_last_error().decode())


def workspace_size(p: Params, call: int) -> int:
    n = ctypes.c_size_t(0)
    check(lib().elsaa_workspace_size(ctypes.byref(p), call, ctypes.byref(n)))
    return int(n.value)


def profile(enable: bool) -> None:
    """Start (discarding earlier records) or stop per-kernel event timing."""
    check(lib().elsaa_profile(1 if enable else 0))


def profile_report() -> dict:
    """{kernel name: (launches, total milliseconds)} of the recorded launches."""
    need = ctypes.c_size_t(0)
    check(lib().elsaa_profile_report(None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(int(need.value) + 16)
    check(lib().elsaa_profile_report(buf, len(buf), ctypes.byref(need)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        out[name] = (int(n), float(ms))
    return out
