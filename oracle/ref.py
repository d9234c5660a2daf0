"""ctypes binding of the ELSAA oracle (TEST INFRASTRUCTURE ONLY).

The oracle is a plain fp64 CPU implementation of the operator of "ELSAA:
Efficient Low-Rank and Sparse Attention Approximation for Training
Transformers" (Sections 3, 3.1, 3.2, 3.3; Eq. 4 and Eq. 5). Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may use it; the
product path never does.

Inputs are numpy arrays holding G independent heads: Q, K, V, dO as float64
[G, N, d]; planes_s float32 [G, hash_bits, d]; planes_lr float32
[G, lr_tables, lr_bits, d]; lam float64 [G]; gates float64 [G, N] or None.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "elsaa_ref.c")
_LIB = os.path.join(_HERE, "libelsaa_ref.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _P(ctypes.Structure):
    _fields_ = [("G", ctypes.c_int), ("N", ctypes.c_int), ("d", ctypes.c_int),
                ("causal", ctypes.c_int), ("block", ctypes.c_int), ("hash_bits", ctypes.c_int),
                ("lr_tables", ctypes.c_int), ("lr_bits", ctypes.c_int), ("chunk", ctypes.c_int),
                ("tau", ctypes.c_double), ("eps", ctypes.c_double), ("scale", ctypes.c_double),
                ("hash_rounds", ctypes.c_int), ("extra_edges", ctypes.c_int)]


@dataclass
class RefParams:
    N: int
    d: int
    causal: bool
    block: int
    hash_bits: int
    lr_tables: int
    lr_bits: int = 4
    chunk: int = 128
    tau: float = 1.0
    eps: float = 1e-6
    scale: float | None = None
    hash_rounds: int = 1
    extra_edges: int = 0   # entries per query of the extra edge list (Omega_safe)

    @property
    def r(self) -> int:
        return self.lr_tables << self.lr_bits

    @property
    def levels(self) -> int:
        return int(round(math.log2(self.N // self.block))) if self.causal else 1

    @classmethod
    def from_workload(cls, w, **kw) -> "RefParams":
        base = dict(N=w.N, d=w.d, causal=w.causal, block=w.block, hash_bits=w.hash_bits,
                    lr_tables=w.lr_tables, lr_bits=w.lr_bits, chunk=w.chunk)
        base.update(kw)
        return cls(**base)

    def c(self, G: int) -> _P:
        sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)
        return _P(G, self.N, self.d, int(self.causal), self.block, self.hash_bits, self.lr_tables,
                  self.lr_bits, self.chunk, self.tau, self.eps, sc, self.hash_rounds,
                  self.extra_edges)


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid parameters (rc={rc})")


def select(p: RefParams, q, k, planes_s):
    """Codes and orders of every head. One round: codes [G, N], orders [G, levels, N/2]
    (causal) or [G, 1, N]; several (planes_s [G, rounds, bits, d]): a round axis after G."""
    q, k, ps = _f64(q), _f64(k), _f32(planes_s)
    G, N = q.shape[0], p.N
    R = max(1, p.hash_rounds)
    plen = p.levels * (N // 2) if p.causal else N
    qc = np.zeros((G, R, N), np.uint16)
    kc = np.zeros((G, R, N), np.uint16)
    qp = np.zeros((G, R, plen), np.int32)
    kp = np.zeros((G, R, plen), np.int32)
    pc = p.c(G)
    _check(lib().ref_select(ctypes.byref(pc), _ptr(q), _ptr(k), _ptr(ps), _ptr(qc), _ptr(kc),
                            _ptr(qp), _ptr(kp)), "select")
    shape = (G, R, p.levels, N // 2) if p.causal else (G, R, 1, N)
    qp, kp = qp.reshape(shape), kp.reshape(shape)
    if R == 1:
        return qc[:, 0], kc[:, 0], qp[:, 0], kp[:, 0]
    return qc, kc, qp, kp


def lowrank_summary(p: RefParams, k, v, planes_lr):
    k, v, pl = _f64(k), _f64(v), _f32(planes_lr)
    G, r, d = k.shape[0], p.r, p.d
    nA = p.N // p.chunk if p.causal else 1
    A = np.zeros((G, nA, r, d))
    z = np.zeros((G, nA, r))
    pc = p.c(G)
    _check(lib().ref_lowrank_summary(ctypes.byref(pc), _ptr(k), _ptr(v), _ptr(pl), _ptr(A), _ptr(z)),
           "lowrank_summary")
    if not p.causal:
        A, z = A[:, 0], z[:, 0]
    return A, z


def _extra(p: RefParams, extra, G):
    if extra is None or p.extra_edges == 0:
        return None
    e = np.ascontiguousarray(np.asarray(extra, dtype=np.int32))
    if e.shape != (G, p.N, p.extra_edges):
        raise ValueError(f"extra has shape {e.shape}, expected {(G, p.N, p.extra_edges)}")
    return e


def forward(p: RefParams, q, k, v, planes_s, planes_lr, lam, g_s=None, g_lr=None, extra=None):
    """extra: int32 [G, N, extra_edges] further keys per query (Omega_safe), or None."""
    q, k, v, ps, pl = _f64(q), _f64(k), _f64(v), _f32(planes_s), _f32(planes_lr)
    lam, g_s, g_lr = _f64(lam), _f64(g_s), _f64(g_lr)
    ex = _extra(p, extra, q.shape[0])
    G, N, d = q.shape
    out = {n: np.zeros((G, N, d)) for n in ("O", "O_s", "O_lr")}
    out.update({n: np.zeros((G, N)) for n in ("lse", "d_lr")})
    pc = p.c(G)
    _check(lib().ref_fwd(ctypes.byref(pc), _ptr(q), _ptr(k), _ptr(v), _ptr(ps), _ptr(pl), _ptr(lam),
                         _ptr(g_s), _ptr(g_lr), _ptr(ex), _ptr(out["O"]), _ptr(out["O_s"]),
                         _ptr(out["O_lr"]),
                         _ptr(out["lse"]), _ptr(out["d_lr"])), "fwd")
    return out


def backward(p: RefParams, q, k, v, do, planes_s, planes_lr, lam, g_s=None, g_lr=None,
             extra=None):
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    ex = _extra(p, extra, q.shape[0])
    ps, pl, lam, g_s, g_lr = _f32(planes_s), _f32(planes_lr), _f64(lam), _f64(g_s), _f64(g_lr)
    G, N, d = q.shape
    out = {n: np.zeros((G, N, d)) for n in ("dQ", "dK", "dV")}
    out["dlambda"] = np.zeros(G)
    out["dg_s"] = np.zeros((G, N))
    out["dg_lr"] = np.zeros((G, N))
    pc = p.c(G)
    _check(lib().ref_bwd(ctypes.byref(pc), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(ps), _ptr(pl),
                         _ptr(lam), _ptr(g_s), _ptr(g_lr), _ptr(ex), _ptr(out["dQ"]), _ptr(out["dK"]),
                         _ptr(out["dV"]), _ptr(out["dlambda"]), _ptr(out["dg_s"]),
                         _ptr(out["dg_lr"])), "bwd")
    return out


def gates_fwd(p: RefParams, q, W, b):
    """Learnable gates g_s, g_lr [G, N] = sigmoid(<W[:, k], Q_i> + b[:, k]), W [G, 2, d],
    b [G, 2]."""
    q, W, b = _f64(q), _f64(W), _f64(b)
    G, N, _ = q.shape
    gs = np.zeros((G, N))
    gl = np.zeros((G, N))
    _check(lib().ref_gates_fwd(ctypes.byref(p.c(G)), _ptr(q), _ptr(W), _ptr(b), _ptr(gs),
                               _ptr(gl)), "gates_fwd")
    return gs, gl


def gates_bwd(p: RefParams, q, W, b, dg_s, dg_lr):
    """The gate path's (dQ, dW, db) from dL/dg_s, dL/dg_lr."""
    q, W, b, dg_s, dg_lr = _f64(q), _f64(W), _f64(b), _f64(dg_s), _f64(dg_lr)
    G, N, d = q.shape
    dq = np.zeros((G, N, d))
    dW = np.zeros((G, 2, d))
    db = np.zeros((G, 2))
    _check(lib().ref_gates_bwd(ctypes.byref(p.c(G)), _ptr(q), _ptr(W), _ptr(b), _ptr(dg_s),
                               _ptr(dg_lr), _ptr(dq), _ptr(dW), _ptr(db)), "gates_bwd")
    return dq, dW, db


def topk(p: RefParams, q, k, k_top: int):
    """Exact per-query top-k keys on Q K^T: int32 [G, N, k_top], ascending, -1 padded."""
    q, k = _f64(q), _f64(k)
    G, N, _ = q.shape
    idx = np.zeros((G, N, k_top), np.int32)
    _check(lib().ref_topk(ctypes.byref(p.c(G)), _ptr(q), _ptr(k), int(k_top), _ptr(idx)), "topk")
    return idx


def features(p: RefParams, planes_lr_head, x):
    """RACE soft bucket assignment phi(x) for rows x [n, d] of one head."""
    x = _f64(x)
    pl = _f32(planes_lr_head)
    out = np.zeros((x.shape[0], p.r))
    pc = p.c(1)
    for t in range(x.shape[0]):
        row = np.ascontiguousarray(x[t])
        o = np.zeros(p.r)
        _check(lib().ref_features(ctypes.byref(pc), _ptr(pl), _ptr(row), _ptr(o)), "features")
        out[t] = o
    return out
