"""Helpers shared by the GPU parity tests: run the oracle and the HIP library on
the same seeded inputs and compare.

Error metric (both dtypes): max |x - ref| / max |ref| over a tensor. Bars:
1e-4 for fp32, 2e-2 for bf16. Codes and permutations are compared exactly."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import ref

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.abs(r).max()
    return float(np.abs(x - r).max() / (den if den > 0 else 1.0))


def cfg_of(w: W.Workload, **kw):
    from sparse_rank_approximation_amd import ElsaaConfig
    return ElsaaConfig(w.B, w.H, w.N, w.d, w.torch_dtype, w.causal, w.block, w.hash_bits,
                       w.lr_tables, w.lr_bits, w.chunk, **kw)


def to_dev(inp: dict, dev="cuda") -> dict:
    return {k: v.to(dev) for k, v in inp.items()}


def head_arrays(w: W.Workload, inp: dict, heads):
    """Oracle inputs (fp64 numpy, exact upcasts) for the listed heads."""
    def take(t):
        return np.stack([t[b, h].double().numpy() for b, h in heads])
    ps = np.stack([inp["planes_s"][h].numpy() for _, h in heads])
    pl = np.stack([inp["planes_lr"][h].numpy() for _, h in heads])
    return take(inp["q"]), take(inp["k"]), take(inp["v"]), take(inp["do"]), ps, pl


def gpu_forward(w, inp, lam, gs=None, glr=None, **cfgkw):
    import sparse_rank_approximation_amd as S
    cfg = cfg_of(w, **cfgkw)
    d = to_dev({k: v for k, v in inp.items()})
    qc, kc, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    A, z = S.lowrank_summary(cfg, d["k"], d["v"], d["planes_lr"])
    lam_d = lam.to("cuda", torch.float32)
    gs_d = None if gs is None else gs.to("cuda", torch.float32).contiguous()
    glr_d = None if glr is None else glr.to("cuda", torch.float32).contiguous()
    out = S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lam_d, gs_d, glr_d)
    torch.cuda.synchronize()
    res = dict(qc=qc, kc=kc, qp=qp, kp=kp, A=A, z=z, **out)
    return cfg, d, res, (lam_d, gs_d, glr_d)


def all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]
