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
    for call in range(7):
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
    (dict(hash_rounds=5), _lib.ERR_UNSUPPORTED, "hash_rounds"),
    (dict(extra_edges=65), _lib.ERR_UNSUPPORTED, "extra_edges"),
    (dict(dtype=torch.bfloat16, d=128, block=256, N=1024, hash_rounds=2), _lib.ERR_UNSUPPORTED,
     "LDS"),
    (dict(B=300, H=300), _lib.ERR_INVALID_ARG, "65535"),
    (dict(B=1, H=100, N=1 << 24, block=16, hash_bits=12, hash_rounds=2), _lib.ERR_INVALID_ARG,
     "2^31"),
    (dict(B=1, H=200, N=1 << 24, block=16, hash_bits=12), _lib.ERR_INVALID_ARG, "2^31"),
])
def test_invalid_parameters(kw, status, needle):
    s, msg, _ = status_of(base(**kw))
    assert s == status, msg
    assert needle in msg


def test_hash_rounds_sizes():
    """Several hash rounds: the orders and the partial slots grow with the rounds;
    0 and 1 both mean one round; a negative count is rejected."""
    one, two = base(), base(hash_rounds=2)
    assert two.perm_len == 2 * one.perm_len
    for call in (_lib.CALL_SELECT, _lib.CALL_FWD, _lib.CALL_BWD):
        s1, m1, n1 = status_of(one, call)
        s2, m2, n2 = status_of(two, call)
        assert s1 == _lib.OK and s2 == _lib.OK, (m1, m2)
        assert n2 > n1, call
    p = one.params()
    p.hash_rounds = 0
    assert status_of(p, _lib.CALL_FWD)[2] == status_of(one, _lib.CALL_FWD)[2]
    p.hash_rounds = -1
    s, msg, _ = status_of(p, _lib.CALL_FWD)
    assert s == _lib.ERR_INVALID_ARG and "hash_rounds" in msg


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
    args = [fake] * 17 + [None, 0, None]  # ws NULL with 0 bytes
    s = L.elsaa_fwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_WORKSPACE, L.elsaa_last_error().decode()
    args = [fake] * 5 + [None] * 12 + [None, 0, None]
    s = L.elsaa_fwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG
    # extra edges: the list is required when extra_edges > 0 (argument 7)
    pe = base(extra_edges=8).params()
    args = [fake] * 17 + [fake, 1 << 40, None]
    args[6] = None
    s = L.elsaa_fwd(ctypes.byref(pe), *args)
    assert s == _lib.ERR_INVALID_ARG and "extra_idx" in L.elsaa_last_error().decode()
    args = [fake] * 23 + [fake, 1 << 40, None]
    args[9] = None
    s = L.elsaa_bwd(ctypes.byref(pe), *args)
    assert s == _lib.ERR_INVALID_ARG and "extra_idx" in L.elsaa_last_error().decode()
    s = L.elsaa_lowrank_summary(ctypes.byref(p), fake, fake, fake, fake, fake, None, 10, None)
    assert s == _lib.ERR_WORKSPACE


def test_check_orders_validates_before_launching():
    L = _lib.lib()
    ok = ctypes.c_void_p(0x1000)
    p = base().params()
    s = L.elsaa_check_orders(ctypes.byref(p), ok, ok, None, ok, 1 << 40, None)
    assert s == _lib.ERR_INVALID_ARG and "bad" in L.elsaa_last_error().decode()
    s = L.elsaa_check_orders(ctypes.byref(p), ok, ok, ok, None, 0, None)
    assert s == _lib.ERR_WORKSPACE
    # the counters: one int32 per token of every head
    n = status_of(base(), _lib.CALL_CHECK)[2]
    assert n == (4 * p.B * p.H * p.N + 255) // 256 * 256


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_misaligned_pointers_are_rejected_before_launching():
    """Every pointer must be 16-byte aligned (the kernels use 16-byte vector
    loads): a misaligned one, required or optional, is INVALID_ARG, and nothing
    is launched (the fake addresses are never dereferenced)."""
    L = _lib.lib()
    p = base().params()
    ok = ctypes.c_void_p(0x1000)
    bad = ctypes.c_void_p(0x1008)
    # elsaa_fwd: Q misaligned
    args = [bad] + [ok] * 16 + [ok, 1 << 40, None]
    s = L.elsaa_fwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG and "aligned" in L.elsaa_last_error().decode()
    # elsaa_fwd: optional gate g_s misaligned (argument 11)
    args = [ok] * 17 + [ok, 1 << 40, None]
    args[10] = bad
    s = L.elsaa_fwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG and "g_s" in L.elsaa_last_error().decode()
    # elsaa_bwd: optional dg_lr misaligned (argument 23)
    args = [ok] * 23 + [ok, 1 << 40, None]
    args[22] = bad
    s = L.elsaa_bwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG and "dg_lr" in L.elsaa_last_error().decode()
    # the workspace too
    args = [ok] * 17 + [bad, 1 << 40, None]
    s = L.elsaa_fwd(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG and "ws" in L.elsaa_last_error().decode()
    s = L.elsaa_select(ctypes.byref(p), ok, ok, ok, ok, bad, ok, ok, ok, 1 << 40, None)
    assert s == _lib.ERR_INVALID_ARG and "k_code" in L.elsaa_last_error().decode()


def test_noalloc_select_rejects_sizes_beyond_its_scratch():
    """elsaa_select_noalloc holds at most 1 MiB of scratch (8 * H * hash_bits * d_h
    bytes): larger sizes are ELSAA_ERR_UNSUPPORTED, checked before any GPU call."""
    L = _lib.lib()
    ok = ctypes.c_void_p(0x1000)
    p = base(H=128, d=128, hash_bits=12, N=1 << 16, block=16).params()  # 1.5 MiB
    s = L.elsaa_select_noalloc(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, None)
    assert s == _lib.ERR_UNSUPPORTED, L.elsaa_last_error().decode()
    assert "at most 1048576 bytes" in L.elsaa_last_error().decode()
    p = base().params()
    s = L.elsaa_select_noalloc(ctypes.byref(p), None, ok, ok, ok, ok, ok, ok, None)
    assert s == _lib.ERR_INVALID_ARG and "NULL" in L.elsaa_last_error().decode()


@pytest.mark.parametrize("kw,needle", [
    (dict(causal=True), "non-causal"),
    (dict(causal=False, hash_rounds=2), "one hash round"),
    (dict(causal=False, extra_edges=4), "extra"),
    (dict(causal=False, N=1 << 16, block=16, hash_bits=12), "hash_bits"),
    (dict(causal=False, N=1 << 16, d=128, lr_tables=8), "LDS"),
])
def test_fused_forward_rejects_what_it_does_not_take(kw, needle):
    """elsaa_fwd_fused takes non-causal, single-round problems without extra edges
    whose head fits one workgroup's LDS; anything else is ELSAA_ERR_UNSUPPORTED,
    decided before any pointer is looked at or anything launched."""
    L = _lib.lib()
    p = base(**kw).params()
    s = L.elsaa_fwd_fused(ctypes.byref(p), *([None] * 20))
    assert s == _lib.ERR_UNSUPPORTED, L.elsaa_last_error().decode()
    assert needle in L.elsaa_last_error().decode()


def test_fused_forward_validates_pointers_before_launching():
    L = _lib.lib()
    ok = ctypes.c_void_p(0x1000)
    bad = ctypes.c_void_p(0x1008)
    p = base(causal=False, N=1024, block=32, lr_tables=2).params()
    args = [ok] * 19 + [None]
    args[8] = None  # q_code
    s = L.elsaa_fwd_fused(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG and "q_code" in L.elsaa_last_error().decode()
    args = [ok] * 19 + [None]
    args[6] = bad  # g_s (optional) misaligned
    s = L.elsaa_fwd_fused(ctypes.byref(p), *args)
    assert s == _lib.ERR_INVALID_ARG and "g_s" in L.elsaa_last_error().decode()
