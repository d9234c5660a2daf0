"""Helpers shared by the GPU parity tests: run the oracle and the HIP library on
the same seeded inputs and compare.

Error metric (both dtypes): max |x - ref| / max |ref| over a tensor; in addition,
per element, the absolute error of lse (the relative error of d_sparse =
exp(lse)) and the relative error of d_lr. Bars: 1e-4 for fp32, 2e-2 for bf16,
the same for every case and every output. Codes and permutations are compared
exactly."""
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


def lse_abs_err(x, r) -> float:
    """Largest |lse - ref| per element: the relative error of d_sparse = exp(lse)."""
    return float(np.abs(np.asarray(x, np.float64) - np.asarray(r, np.float64)).max())


def elem_rel_err(x, r) -> float:
    """Largest |x - ref| / |ref| per element (for a strictly positive ref, d_lr)."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    return float((np.abs(x - r) / np.abs(r)).max())


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


def wl(name, B, H, N, d, dtype, causal, block, r, gen="iid", chunk=128, **ga):
    return W.Workload(name, B, H, N, d, dtype, causal, block, r, gen, ga, chunk=chunk)

CASES = {
    # the tiny single-head workload, as is
    "tiny_f32": (W.WORKLOADS[1], False, False),
    # several tiles and summary chunks, causal, fp32
    "causal_f32_N512_d64_s32": (wl("c", 1, 2, 512, 64, "f32", True, 32, 32, chunk=128), True, True),
    # bf16 causal with planted clusters, d 128, s 128, r 128, two summaries per head
    "causal_bf16_N1024_d128_s128": (wl("c", 1, 2, 1024, 128, "bf16", True, 128, 128,
                                       "clusters", chunk=512, n_clusters=16, sigma=0.5), True, True),
    # bf16 causal, d 64, s 128: the backward's 16-key-tile kernel at d 64 over the
    # off-diagonal levels as well as the leaves
    "causal_bf16_N1024_d64_s128": (wl("c", 1, 2, 1024, 64, "bf16", True, 128, 64,
                                      "clusters", chunk=256, n_clusters=16, sigma=0.5), True, True),
    # bf16 non-causal, d 128, s 128, three blocks per head and three heads (a block
    # count that is no multiple of the eight XCDs)
    "noncausal_bf16_N384_d128_s128": (wl("n", 1, 3, 384, 128, "bf16", False, 128, 64,
                                         "clusters", n_clusters=8, sigma=0.5), True, True),
    # bf16 non-causal vision-like field, d 64, s 32, r 32
    "vit_bf16_N1024_d64_s32": (wl("v", 2, 2, 1024, 64, "bf16", False, 32, 32, "smooth_field",
                                  grid=32, blur=2.0, noise=0.3), False, False),
    # ragged: 96 tokens = one 64-token step plus a 32-token tail; 3 blocks of 32
    "ragged_noncausal_f32_N96": (wl("r", 1, 1, 96, 32, "f32", False, 32, 16), True, True),
    # ragged causal: 32-token summary chunks inside 64-token steps; block 16
    "ragged_causal_f32_N256_s16_chunk32": (wl("r", 1, 1, 256, 32, "f32", True, 16, 48, chunk=32),
                                           True, False),
    # degenerate causal: N == block, no off-diagonal level (dense causal softmax)
    "causal_single_block_f32": (wl("d", 1, 1, 64, 32, "f32", True, 64, 32, chunk=64), False, False),
    # the same in bf16 (empty orders, passed as null pointers), two heads
    "causal_single_block_bf16": (wl("e", 1, 2, 128, 64, "bf16", True, 128, 32, chunk=128),
                                 True, True),
    # peaked softmax: 128 tight clusters of 4 tokens at d 128, so a query's few
    # same-cluster keys (scores near 11, the rest near 0) often sit in a later key
    # tile than the first and the sparse forward's running maximum has to move
    "peaked_clusters_bf16_causal": (wl("k", 1, 2, 512, 128, "bf16", True, 128, 32, "clusters",
                                       chunk=128, n_clusters=128, sigma=0.1), True, True),
    # odd table count (padded to 4 tables on the GPU), bf16, d 32
    "tables3_bf16_causal": (wl("t", 1, 1, 512, 32, "bf16", True, 64, 48, chunk=256), True, True),
    # maximum block 256 and r 256 at d 128, causal bf16
    "block256_bf16": (wl("m", 1, 1, 1024, 128, "bf16", True, 256, 256, "clusters", chunk=512,
                         n_clusters=8, sigma=0.5), False, False),
}
