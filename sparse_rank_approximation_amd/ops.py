"""Python surface of libelsaa: the four C calls with torch device tensors, and
an autograd Function over them.

PyTorch provides device memory and the current stream only; argument
marshalling happens here, every computation in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, replace

import torch

from . import _lib


@dataclass(frozen=True)
class ElsaaConfig:
    """Problem sizes and method parameters (see include/elsaa.h, elsaa_params)."""
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype = torch.bfloat16
    causal: bool = False
    block: int = 128          # sortLSH block size s
    hash_bits: int | None = None  # default log2(N / block), at least 1
    lr_tables: int = 8        # RACE tables L (r = 16 L features)
    lr_bits: int = 4
    chunk: int = 2048         # causal RACE summary spacing (rounding only; larger is faster)
    tau: float = 1.0
    eps: float = 1e-6
    scale: float | None = None
    hash_rounds: int = 1      # sortLSH hash tables (support = union over the rounds)
    extra_edges: int = 0      # keys listed per query joining the sparse support

    @property
    def bits(self) -> int:
        if self.hash_bits is not None:
            return self.hash_bits
        return max(1, int(round(math.log2(max(1, self.N // self.block)))))

    @property
    def r(self) -> int:
        return self.lr_tables << self.lr_bits

    @property
    def levels(self) -> int:
        return int(round(math.log2(self.N // self.block))) if self.causal else 1

    @property
    def rounds(self) -> int:
        return max(1, self.hash_rounds)

    @property
    def perm_len(self) -> int:
        return self.rounds * (self.levels * (self.N // 2) if self.causal else self.N)

    @property
    def planes_s_shape(self) -> tuple:
        """[H, bits, d] with one round, [H, R, bits, d] with several."""
        if self.rounds == 1:
            return (self.H, self.bits, self.d)
        return (self.H, self.rounds, self.bits, self.d)

    @property
    def code_shape(self) -> tuple:
        """[B, H, N] with one round, [B, H, R, N] with several."""
        if self.rounds == 1:
            return (self.B, self.H, self.N)
        return (self.B, self.H, self.rounds, self.N)

    @property
    def n_summaries(self) -> int:
        return self.N // self.eff_chunk if self.causal else 1

    @property
    def eff_chunk(self) -> int:
        return min(self.chunk, self.N)

    def with_(self, **kw) -> "ElsaaConfig":
        return replace(self, **kw)

    def params(self) -> _lib.Params:
        if self.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError(f"dtype {self.dtype} is not supported (float32 or bfloat16)")
        sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)
        return _lib.Params(self.B, self.H, self.N, self.d,
                           _lib.BF16 if self.dtype == torch.bfloat16 else _lib.F32,
                           int(self.causal), self.block, self.bits, self.lr_tables, self.lr_bits,
                           self.eff_chunk, self.tau, self.eps, sc, self.rounds, self.extra_edges)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(name, t, shape, dtype, device):
    if t is not None:
        _check_tensor(name, t, shape, dtype, device)
    return t


def _workspace(cfg: ElsaaConfig, call: int, device) -> tuple[torch.Tensor | None, int]:
    n = _lib.workspace_size(cfg.params(), call)
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def select(cfg: ElsaaConfig, q, k, planes_s):
    """elsaa_select: codes [B,H,N] ([B,H,R,N] with R > 1 hash rounds) uint16 (as int16
    storage) and perms [B,H,P] int32."""
    dev = q.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    _check_tensor("q", q, x, cfg.dtype, dev)
    _check_tensor("k", k, x, cfg.dtype, dev)
    _check_tensor("planes_s", planes_s, cfg.planes_s_shape, torch.float32, dev)
    qc = torch.empty(cfg.code_shape, dtype=torch.int16, device=dev)
    kc = torch.empty_like(qc)
    qp = torch.empty(cfg.B, cfg.H, cfg.perm_len, dtype=torch.int32, device=dev)
    kp = torch.empty_like(qp)
    ws, n = _workspace(cfg, _lib.CALL_SELECT, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_select(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(planes_s),
                                       _ptr(qc), _ptr(kc), _ptr(qp) if qp.numel() else None,
                                       _ptr(kp) if kp.numel() else None, _ptr(ws), n,
                                       _stream(dev)))
    return qc, kc, qp, kp


def select_noalloc(cfg: ElsaaConfig, q, k, planes_s, out=None):
    """elsaa_select_noalloc: the same selection with no workspace. `out` =
    (q_code, k_code, q_perm, k_perm) preallocated by the caller, or None to have
    them allocated here (the call itself allocates nothing)."""
    dev = q.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    _check_tensor("q", q, x, cfg.dtype, dev)
    _check_tensor("k", k, x, cfg.dtype, dev)
    _check_tensor("planes_s", planes_s, cfg.planes_s_shape, torch.float32, dev)
    if out is None:
        qc = torch.empty(cfg.code_shape, dtype=torch.int16, device=dev)
        qp = torch.empty(cfg.B, cfg.H, cfg.perm_len, dtype=torch.int32, device=dev)
        out = (qc, torch.empty_like(qc), qp, torch.empty_like(qp))
    qc, kc, qp, kp = out
    for name, t, shp, dt in (("q_code", qc, cfg.code_shape, torch.int16),
                             ("k_code", kc, cfg.code_shape, torch.int16),
                             ("q_perm", qp, (cfg.B, cfg.H, cfg.perm_len), torch.int32),
                             ("k_perm", kp, (cfg.B, cfg.H, cfg.perm_len), torch.int32)):
        _check_tensor(name, t, shp, dt, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_select_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(planes_s),
                                               _ptr(qc), _ptr(kc),
                                               _ptr(qp) if qp.numel() else None,
                                               _ptr(kp) if kp.numel() else None, _stream(dev)))
    return qc, kc, qp, kp


def check_orders(cfg: ElsaaConfig, q_perm, k_perm):
    """elsaa_check_orders: int32 [B, H], the number of entries of each head's orders
    that break the order layout (0 for orders elsaa_select wrote)."""
    dev = q_perm.device
    _check_tensor("q_perm", q_perm, (cfg.B, cfg.H, cfg.perm_len), torch.int32, dev)
    _check_tensor("k_perm", k_perm, (cfg.B, cfg.H, cfg.perm_len), torch.int32, dev)
    bad = torch.empty(cfg.B, cfg.H, dtype=torch.int32, device=dev)
    ws, n = _workspace(cfg, _lib.CALL_CHECK, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_check_orders(ctypes.byref(p),
                                             _ptr(q_perm) if q_perm.numel() else None,
                                             _ptr(k_perm) if k_perm.numel() else None,
                                             _ptr(bad), _ptr(ws), n, _stream(dev)))
    return bad


def topk(cfg: ElsaaConfig, q, k, k_top: int):
    """elsaa_topk: exact per-query top-k keys on Q K^T, int32 [B,H,N,k_top] ascending,
    -1 padded (causal: keys j <= i)."""
    dev = q.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    _check_tensor("q", q, x, cfg.dtype, dev)
    _check_tensor("k", k, x, cfg.dtype, dev)
    idx = torch.empty(cfg.B, cfg.H, cfg.N, k_top, dtype=torch.int32, device=dev)
    ws, n = _workspace(cfg, _lib.CALL_TOPK, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_topk(ctypes.byref(p), _ptr(q), _ptr(k), int(k_top), _ptr(idx),
                                     _ptr(ws), n, _stream(dev)))
    return idx


def lowrank_summary(cfg: ElsaaConfig, k, v, planes_lr):
    """elsaa_lowrank_summary: A [B,H,nA,d,r], z [B,H,nA,r] fp32."""
    dev = k.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    _check_tensor("k", k, x, cfg.dtype, dev)
    _check_tensor("v", v, x, cfg.dtype, dev)
    _check_tensor("planes_lr", planes_lr, (cfg.H, cfg.lr_tables, cfg.lr_bits, cfg.d),
                  torch.float32, dev)
    nA = cfg.n_summaries
    A = torch.empty(cfg.B, cfg.H, nA, cfg.d, cfg.r, dtype=torch.float32, device=dev)
    z = torch.empty(cfg.B, cfg.H, nA, cfg.r, dtype=torch.float32, device=dev)
    ws, n = _workspace(cfg, _lib.CALL_SUMMARY, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_lowrank_summary(ctypes.byref(p), _ptr(k), _ptr(v),
                                                _ptr(planes_lr), _ptr(A), _ptr(z), _ptr(ws), n,
                                                _stream(dev)))
    return A, z


def _extra_idx(cfg: ElsaaConfig, extra, dev):
    if cfg.extra_edges == 0:
        if extra is not None:
            raise ValueError("extra edges given but cfg.extra_edges is 0")
        return None
    _check_tensor("extra", extra, (cfg.B, cfg.H, cfg.N, cfg.extra_edges), torch.int32, dev)
    return extra


def forward(cfg: ElsaaConfig, q, k, v, planes_lr, q_perm, k_perm, A, z, lam, g_s=None, g_lr=None,
            extra=None):
    """elsaa_fwd: returns dict(O, O_s (fp32), O_lr, lse, d_lr). extra: int32
    [B,H,N,extra_edges] keys per query joining the sparse support (-1 padded)."""
    dev = q.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, x, cfg.dtype, dev)
    _check_tensor("planes_lr", planes_lr, (cfg.H, cfg.lr_tables, cfg.lr_bits, cfg.d),
                  torch.float32, dev)
    _check_tensor("q_perm", q_perm, (cfg.B, cfg.H, cfg.perm_len), torch.int32, dev)
    _check_tensor("k_perm", k_perm, (cfg.B, cfg.H, cfg.perm_len), torch.int32, dev)
    _check_tensor("A", A, (cfg.B, cfg.H, cfg.n_summaries, cfg.d, cfg.r), torch.float32, dev)
    _check_tensor("z", z, (cfg.B, cfg.H, cfg.n_summaries, cfg.r), torch.float32, dev)
    _check_tensor("lam", lam, (cfg.H,), torch.float32, dev)
    _opt("g_s", g_s, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    _opt("g_lr", g_lr, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    extra = _extra_idx(cfg, extra, dev)
    out = {n: torch.empty(x, dtype=cfg.dtype, device=dev) for n in ("O", "O_lr")}
    out["O_s"] = torch.empty(x, dtype=torch.float32, device=dev)
    out["lse"] = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev)
    out["d_lr"] = torch.empty_like(out["lse"])
    ws, n = _workspace(cfg, _lib.CALL_FWD, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_fwd(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(planes_lr),
        _ptr(q_perm) if q_perm.numel() else None, _ptr(k_perm) if k_perm.numel() else None,
        _ptr(extra), _ptr(A), _ptr(z), _ptr(lam), _ptr(g_s), _ptr(g_lr), _ptr(out["O"]),
        _ptr(out["O_s"]),
        _ptr(out["O_lr"]), _ptr(out["lse"]), _ptr(out["d_lr"]), _ptr(ws), n, _stream(dev)))
    return out


def forward_fused(cfg: ElsaaConfig, q, k, v, planes_s, planes_lr, lam, g_s=None, g_lr=None):
    """elsaa_fwd_fused: the non-causal forward in one launch. Returns dict(q_code, k_code,
    q_perm, k_perm, A, z, O, O_s, O_lr, lse, d_lr), what select, lowrank_summary and
    forward return together (and what backward takes)."""
    dev = q.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, x, cfg.dtype, dev)
    _check_tensor("planes_s", planes_s, cfg.planes_s_shape, torch.float32, dev)
    _check_tensor("planes_lr", planes_lr, (cfg.H, cfg.lr_tables, cfg.lr_bits, cfg.d),
                  torch.float32, dev)
    _check_tensor("lam", lam, (cfg.H,), torch.float32, dev)
    _opt("g_s", g_s, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    _opt("g_lr", g_lr, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    out = {"q_code": torch.empty(cfg.code_shape, dtype=torch.int16, device=dev)}
    out["k_code"] = torch.empty_like(out["q_code"])
    out["q_perm"] = torch.empty(cfg.B, cfg.H, cfg.perm_len, dtype=torch.int32, device=dev)
    out["k_perm"] = torch.empty_like(out["q_perm"])
    out["A"] = torch.empty(cfg.B, cfg.H, cfg.n_summaries, cfg.d, cfg.r, dtype=torch.float32,
                           device=dev)
    out["z"] = torch.empty(cfg.B, cfg.H, cfg.n_summaries, cfg.r, dtype=torch.float32, device=dev)
    for n in ("O", "O_lr"):
        out[n] = torch.empty(x, dtype=cfg.dtype, device=dev)
    out["O_s"] = torch.empty(x, dtype=torch.float32, device=dev)
    out["lse"] = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev)
    out["d_lr"] = torch.empty_like(out["lse"])
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_fwd_fused(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(planes_s), _ptr(planes_lr), _ptr(lam),
        _ptr(g_s), _ptr(g_lr), _ptr(out["q_code"]), _ptr(out["k_code"]), _ptr(out["q_perm"]),
        _ptr(out["k_perm"]), _ptr(out["A"]), _ptr(out["z"]), _ptr(out["O"]), _ptr(out["O_s"]),
        _ptr(out["O_lr"]), _ptr(out["lse"]), _ptr(out["d_lr"]), _stream(dev)))
    return out


def backward(cfg: ElsaaConfig, q, k, v, do, O_s, O_lr, planes_lr, q_perm, k_perm, A, z, lse, d_lr,
             lam, g_s=None, g_lr=None, want_dlam=True, want_dg=True, extra=None):
    """elsaa_bwd: returns dict(dQ, dK, dV, dlambda, dg_s, dg_lr)."""
    dev = q.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do), ("O_lr", O_lr)):
        _check_tensor(name, t, x, cfg.dtype, dev)
    _check_tensor("O_s", O_s, x, torch.float32, dev)
    _check_tensor("q_perm", q_perm, (cfg.B, cfg.H, cfg.perm_len), torch.int32, dev)
    _check_tensor("k_perm", k_perm, (cfg.B, cfg.H, cfg.perm_len), torch.int32, dev)
    _check_tensor("lse", lse, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    _check_tensor("d_lr", d_lr, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    _check_tensor("lam", lam, (cfg.H,), torch.float32, dev)
    _opt("g_s", g_s, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    _opt("g_lr", g_lr, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    extra = _extra_idx(cfg, extra, dev)
    out = {n: torch.empty(x, dtype=cfg.dtype, device=dev) for n in ("dQ", "dK", "dV")}
    out["dlambda"] = torch.empty(cfg.H, dtype=torch.float32, device=dev) if want_dlam else None
    out["dg_s"] = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev) if want_dg else None
    out["dg_lr"] = torch.empty_like(out["dg_s"]) if want_dg else None
    ws, n = _workspace(cfg, _lib.CALL_BWD, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_bwd(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(O_s), _ptr(O_lr),
        _ptr(planes_lr), _ptr(q_perm) if q_perm.numel() else None,
        _ptr(k_perm) if k_perm.numel() else None, _ptr(extra), _ptr(A), _ptr(z), _ptr(lse),
        _ptr(d_lr),
        _ptr(lam), _ptr(g_s), _ptr(g_lr), _ptr(out["dQ"]), _ptr(out["dK"]), _ptr(out["dV"]),
        _ptr(out["dlambda"]), _ptr(out["dg_s"]), _ptr(out["dg_lr"]), _ptr(ws), n,
        _stream(dev)))
    return out


def gates(cfg: ElsaaConfig, q, W, b):
    """elsaa_gates_fwd: g_s, g_lr [B,H,N] fp32 = sigmoid(<W[h,k], Q_i> + b[h,k])."""
    dev = q.device
    _check_tensor("q", q, (cfg.B, cfg.H, cfg.N, cfg.d), cfg.dtype, dev)
    _check_tensor("W", W, (cfg.H, 2, cfg.d), torch.float32, dev)
    _check_tensor("b", b, (cfg.H, 2), torch.float32, dev)
    gs = torch.empty(cfg.B, cfg.H, cfg.N, dtype=torch.float32, device=dev)
    gl = torch.empty_like(gs)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_gates_fwd(ctypes.byref(p), _ptr(q), _ptr(W), _ptr(b), _ptr(gs),
                                          _ptr(gl), _stream(dev)))
    return gs, gl


def gates_backward(cfg: ElsaaConfig, q, W, g_s, g_lr, dg_s, dg_lr, dq):
    """elsaa_gates_bwd: adds the gate path's gradient to dq (in place) and returns
    (dW [H,2,d], db [H,2])."""
    dev = q.device
    x = (cfg.B, cfg.H, cfg.N, cfg.d)
    _check_tensor("q", q, x, cfg.dtype, dev)
    _check_tensor("dq", dq, x, cfg.dtype, dev)
    _check_tensor("W", W, (cfg.H, 2, cfg.d), torch.float32, dev)
    for name, t in (("g_s", g_s), ("g_lr", g_lr), ("dg_s", dg_s), ("dg_lr", dg_lr)):
        _check_tensor(name, t, (cfg.B, cfg.H, cfg.N), torch.float32, dev)
    dW = torch.empty(cfg.H, 2, cfg.d, dtype=torch.float32, device=dev)
    db = torch.empty(cfg.H, 2, dtype=torch.float32, device=dev)
    ws, n = _workspace(cfg, _lib.CALL_GATES_BWD, dev)
    p = cfg.params()
    _lib.check(_lib.lib().elsaa_gates_bwd(ctypes.byref(p), _ptr(q), _ptr(W), _ptr(g_s), _ptr(g_lr),
                                          _ptr(dg_s), _ptr(dg_lr), _ptr(dq), _ptr(dW), _ptr(db),
                                          _ptr(ws), n, _stream(dev)))
    return dW, db


class ElsaaFunction(torch.autograd.Function):
    """O = ELSAA(Q, K, V; lambda, g_s, g_lr) with gradients for Q, K, V, lambda and
    the gates; the hyperplanes are fixed inputs (no gradient). With gate_w, gate_b
    given, the gates are learned: g = sigmoid(<gate_w[h, k], Q_i> + gate_b[h, k])
    (elsaa_gates_fwd), and gate_w, gate_b get gradients (g_s, g_lr must be None).
    extra: int32 [B, H, N, cfg.extra_edges] keys per query joining the sparse
    support, or None."""

    @staticmethod
    def forward(ctx, cfg, q, k, v, lam, g_s, g_lr, planes_s, planes_lr, gate_w=None, gate_b=None,
                extra=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        learned = gate_w is not None
        if learned:
            if g_s is not None or g_lr is not None:
                raise ValueError("give either gate tensors or a gate projection, not both")
            g_s, g_lr = gates(cfg, q, gate_w.contiguous(), gate_b.contiguous())
        out = None
        if not cfg.causal and cfg.rounds == 1 and extra is None:
            # the one-launch forward where it takes the sizes
            try:
                out = forward_fused(cfg, q, k, v, planes_s, planes_lr, lam, g_s, g_lr)
                qp, kp, A, z = out["q_perm"], out["k_perm"], out["A"], out["z"]
            except _lib.ElsaaError as e:
                if e.status != _lib.ERR_UNSUPPORTED:
                    raise
        if out is None:
            _, _, qp, kp = select(cfg, q, k, planes_s)
            A, z = lowrank_summary(cfg, k, v, planes_lr)
            out = forward(cfg, q, k, v, planes_lr, qp, kp, A, z, lam, g_s, g_lr, extra=extra)
        ctx.cfg = cfg
        ctx.learned = learned
        ctx.save_for_backward(q, k, v, lam, g_s, g_lr, planes_lr, qp, kp, A, z, out["O_s"],
                              out["O_lr"], out["lse"], out["d_lr"],
                              gate_w.contiguous() if learned else None, extra)
        return out["O"]

    @staticmethod
    def backward(ctx, dO):
        (q, k, v, lam, g_s, g_lr, planes_lr, qp, kp, A, z, O_s, O_lr, lse, d_lr,
         gate_w, extra) = ctx.saved_tensors
        want_dg = ctx.learned or ctx.needs_input_grad[5] or ctx.needs_input_grad[6]
        g = backward(ctx.cfg, q, k, v, dO.contiguous(), O_s, O_lr, planes_lr, qp, kp, A, z, lse,
                     d_lr, lam, g_s, g_lr, want_dlam=ctx.needs_input_grad[4], want_dg=want_dg,
                     extra=extra)
        dW = db = None
        if ctx.learned:
            dW, db = gates_backward(ctx.cfg, q, gate_w, g_s, g_lr, g["dg_s"], g["dg_lr"], g["dQ"])
            return (None, g["dQ"], g["dK"], g["dV"], g["dlambda"], None, None, None, None, dW, db,
                    None)
        return (None, g["dQ"], g["dK"], g["dV"], g["dlambda"],
                g["dg_s"] if ctx.needs_input_grad[5] else None,
                g["dg_lr"] if ctx.needs_input_grad[6] else None, None, None, None, None, None)


def make_planes(cfg: ElsaaConfig, seed: int = 0, device="cuda"):
    """iid N(0,1) sortLSH and RACE hyperplanes for every head (fixed, no gradient)."""
    g = torch.Generator().manual_seed(seed)
    ps = torch.randn(*cfg.planes_s_shape, generator=g)
    pl = torch.randn(cfg.H, cfg.lr_tables, cfg.lr_bits, cfg.d, generator=g)
    return ps.to(device), pl.to(device)


def elsaa_attention(q, k, v, *, causal: bool, block: int, lr_tables: int, lam=None, g_s=None,
                    g_lr=None, planes_s=None, planes_lr=None, seed: int = 0, chunk: int = 2048,
                    hash_bits: int | None = None, tau: float = 1.0, eps: float = 1e-6,
                    gate_w=None, gate_b=None, hash_rounds: int = 1, extra_idx=None):
    """ELSAA attention of q, k, v [B, H, N, d] (fp32 or bf16 device tensors). Gates:
    fixed tensors g_s, g_lr [B, H, N], or learned from the projection gate_w [H, 2, d],
    gate_b [H, 2] of the query. extra_idx: int32 [B, H, N, E] keys per query that join
    the sparse support (e.g. random edges, or topk()'s picks), -1 padded."""
    B, H, N, d = q.shape
    cfg = ElsaaConfig(B, H, N, d, q.dtype, causal, block, hash_bits, lr_tables, 4, chunk, tau, eps,
                      hash_rounds=hash_rounds,
                      extra_edges=0 if extra_idx is None else int(extra_idx.shape[-1]))
    if planes_s is None or planes_lr is None:
        ps, pl = make_planes(cfg, seed, q.device)
        planes_s = ps if planes_s is None else planes_s
        planes_lr = pl if planes_lr is None else planes_lr
    if lam is None:
        lam = torch.ones(H, dtype=torch.float32, device=q.device)
    return ElsaaFunction.apply(cfg, q, k, v, lam, g_s, g_lr, planes_s, planes_lr, gate_w, gate_b,
                               extra_idx)
