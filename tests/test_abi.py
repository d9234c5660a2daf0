"""CPU tests of the C ABI: the library loads, exports every function include/elsaa.h
declares, the ctypes declarations match the header's parameter lists, and every
validation error path returns its status and a message without touching a GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

from sparse_rank_approximation_amd import ElsaaConfig, _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "elsaa.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(elsaa_status|const char\*)\s+(elsaa_\w+)\s*\(([^)]*)\)\s*;", src):
        args = [a.strip() for a in m.group(3).split(",") if a.strip() and a.strip() != "void"]
        out[m.group(2)] = args
    return out


def test_header_declares_the_four_calls():
    fns = header_functions()
    for name in ("elsaa_select", "elsaa_lowrank_summary", "elsaa_fwd", "elsaa_bwd",
                 "elsaa_workspace_size", "elsaa_last_error"):
        assert name in fns, name
    assert set(fns) == set(_lib.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in header_functions():
        assert hasattr(L, name), name


def test_ctypes_argument_counts_match_header():
    L = _lib.lib()
    for name, args in header_functions().items():
        assert len(getattr(L, name).argtypes) == len(args), name


def base(**kw):
    c = dict(B=2, H=3, N=1024, d=64, dtype=torch.bfloat16, causal=True, block=64, lr_tables=4,
             chunk=256)
    c.update(kw)
    return ElsaaConfig(**c)


def status_of(cfg_or_params, call=_lib.CALL_FWD):
    p = cfg_or_params.params() if isinstance(cfg_or_params, ElsaaConfig) else cfg_or_params
    n = ctypes.c_size_t(0)
    s = _lib.lib().elsaa_workspace_size(ctypes.byref(p), call, ctypes.byref(n))
    return s, _lib.lib().elsaa_last_error().decode(), n.value


def test_valid_params_and_workspace_sizes():
    for call in range(4):
        s, msg, n = status_of(base(), call)
        assert s == _lib.OK, msg
    # select: the hyperplanes widened to fp64, [H, hash_bits, d_h], 256-byte rounded
    p = base().params()
    assert status_of(base(), _lib.CALL_SELECT)[2] == (8 * p.H * p.hash_bits * p.d_h + 255) // 256 * 256
    assert status_of(base(), _lib.CALL_FWD)[2] > 0
    # An empty batch is valid and needs no workspace.
    assert status_of(base(B=0), _lib.CALL_FWD)[:1] == (_lib.OK,)
    assert status_of(base(B=0), _lib.CALL_FWD)[2] == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(d=48), _lib.ERR_UNSUPPORTED, "d_h"),
    (dict(N=1000), _lib.ERR_INVALID_ARG, "multiple of 32"),
    (dict(block=48), _lib.ERR_UNSUPPORTED, "block"),
    (dict(N=96 * 32, block=32, causal=True), _lib.ERR_INVALID_ARG, "power of two"),
    (dict(N=96, block=64, causal=False), _lib.ERR_INVALID_ARG, "multiple of block"),
    (dict(hash_bits=0), _lib.ERR_INVALID_ARG, "hash_bits"),
    (dict(hash_bits=14), _lib.ERR_UNSUPPORTED, "hash_bits"),
    (dict(lr_tables=0), _lib.ERR_INVALID_ARG, "lr_tables"),
    (dict(lr_tables=17), _lib.ERR_UNSUPPORTED, "lr_tables"),
    (dict(lr_bits=3), _lib.ERR_UNSUPPORTED, "lr_bits"),
    (dict(chunk=48), _lib.ERR_INVALID_ARG, "chunk"),
    (dict(tau=0.0), _lib.ERR_INVALID_ARG, "tau"),
    (dict(eps=-1.0), _lib.ERR_INVALID_ARG, "eps"),
    (dict(scale=float("nan")), _lib.ERR_INVALID_ARG, "scale"),
    (dict(dtype=torch.float32, d=128, block=256, N=1024), _lib.ERR_UNSUPPORTED, "LDS"),
    (dict(B=300, H=300), _lib.ERR_INVALID_ARG, "65535"),
    (dict(B=1, H=200, N=1 << 24, block=16, hash_bits=12), _lib.ERR_INVALID_ARG, "2^31"),
])
def test_invalid_parameters(kw, status, needle):
    s, msg, _ = status_of(base(**kw))
    assert s == status, msg
    assert needle in msg


def test_bad_dtype_and_null_params():
    p = base().params()
    p.dtype = 7
    s, msg, _ = status_of(p)
    assert s == _lib.ERR_INVALID_ARG and "dtype" in msg
    n = ctypes.c_size_t(0)
    assert _lib.lib().elsaa_workspace_size(None, 0, ctypes.byref(n)) == _lib.ERR_INVALID_ARG
    assert _lib.lib().elsaa_workspace_size(ctypes.byref(base().params()), 9,
                                           ctypes.byref(n)) == _lib.ERR_INVALID_ARG


def test_calls_reject_null_pointers_and_short_workspace_before_launching():
    L = _lib.lib()
    p = base().params()
    s = L.elsaa_select(ctypes.byref(p), None, None, None, None, None, None, None, None, 0, None)
    assert s == _lib.ERR_INVALID_ARG and "NULL" in L.elsaa_last_error().decode()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    args = [fake] * 16 + [None, 0, None]  # ws NULL with 0 bytes
    s = L.elsaa_fwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_WORKSPACE, L.elsaa_last_error().decode()
    args = [fake] * 5 + [None] * 11 + [None, 0, None]
    s = L.elsaa_fwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG
    s = L.elsaa_lowrank_summary(ctypes.byref(p), fake, fake, fake, fake, fake, None, 10, None)
    assert s == _lib.ERR_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()
