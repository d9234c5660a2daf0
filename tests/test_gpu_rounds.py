"""GPU parity of several sortLSH hash rounds (the L_s hash tables of Appendix C:
each round hashes with its own hyperplanes and sorts on its own, and a query's
sparse support is the union Omega_LSH of the rounds' supports, every pair
counted once) against the oracle.

Each case runs select, the low-rank summary, the forward and the backward
through the C ABI: codes and orders must match the oracle's exactly, every
output and gradient within the usual bars (1e-4 fp32, 2e-2 bf16, max-relative;
lse per element absolute, d_lr per element relative). A last case hashes twice
with the same hyperplanes: the second round then adds no pair, and the result
must match the one-round call's up to rounding."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from parity_util import (TOL, all_heads, cfg_of, elem_rel_err, head_arrays, lse_abs_err, rel_err,
                         to_dev, wl)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

# name: (workload, rounds)
CASES = {
    # the headline shape on a smaller N: bf16, d 128, blocks of 128, clusters
    "causal_bf16_N1024_d128_s128_R2": (wl("c", 1, 2, 1024, 128, "bf16", True, 128, 128,
                                          "clusters", chunk=512, n_clusters=16, sigma=0.5), 2),
    "causal_f32_N512_d64_s32_R3": (wl("c", 1, 2, 512, 64, "f32", True, 32, 32, chunk=128), 3),
    # blocks of 16 (half-empty key tiles), four rounds
    "causal_bf16_N256_d32_s16_R4": (wl("c", 1, 1, 256, 32, "bf16", True, 16, 32, chunk=64), 4),
    # no off-diagonal level: every round's orders are empty, the leaves hold all pairs
    "causal_single_block_f32_R2": (wl("d", 1, 1, 64, 32, "f32", True, 64, 32, chunk=64), 2),
    "noncausal_bf16_N1024_d64_s64_R2": (wl("n", 2, 1, 1024, 64, "bf16", False, 64, 64,
                                           "clusters_diffuse", n_clusters=16, sigma=0.5,
                                           diffuse=0.2), 2),
    # ragged: 96 tokens, 3 blocks of 32
    "noncausal_f32_N96_d32_s32_R3": (wl("r", 1, 1, 96, 32, "f32", False, 32, 16), 3),
    # blocks of 256 (the key-wave / query-wave launch pair), fp32
    "noncausal_f32_N512_d32_s256_R2": (wl("n", 1, 1, 512, 32, "f32", False, 256, 32), 2),
}


def _run_gpu(w, inp, rounds, lam, gs, glr):
    import sparse_rank_approximation_amd as S
    cfg = cfg_of(w, hash_rounds=rounds)
    d = to_dev(inp)
    qc, kc, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    A, z = S.lowrank_summary(cfg, d["k"], d["v"], d["planes_lr"])
    lam_d = lam.to("cuda", torch.float32)
    gs_d = gs.to("cuda", torch.float32).contiguous()
    glr_d = glr.to("cuda", torch.float32).contiguous()
    f = S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lam_d, gs_d, glr_d)
    g = S.backward(cfg, d["q"], d["k"], d["v"], d["do"], f["O_s"], f["O_lr"], d["planes_lr"], qp, kp,
                   A, z, f["lse"], f["d_lr"], lam_d, gs_d, glr_d)
    torch.cuda.synchronize()
    return dict(qc=qc, kc=kc, qp=qp, kp=kp, **f), g


@pytest.mark.parametrize("case", list(CASES))
def test_rounds_parity(case):
    w, R = CASES[case]
    seed = 4100 + len(case)
    print(f"[gpu rounds] {case} {w} R={R}", flush=True)
    inp = W.gen_inputs(w, seed)
    inp["planes_s"] = W.gen_planes_rounds(w, seed, R)
    lam = W.gen_lambda(w, seed, random=True)
    gs, glr = W.gen_gates(w, seed)
    f, g = _run_gpu(w, inp, R, lam, gs, glr)

    heads = all_heads(w)
    G = len(heads)
    q, k, v, do, ps, pl = head_arrays(w, inp, heads)
    p = ref.RefParams.from_workload(w, hash_rounds=R)
    lamh = np.array([float(lam[h]) for _, h in heads])
    gsh = np.stack([gs[b, h].double().numpy() for b, h in heads])
    glh = np.stack([glr[b, h].double().numpy() for b, h in heads])
    rqc, rkc, rqp, rkp = ref.select(p, q, k, ps)
    np.testing.assert_array_equal(f["qc"].view(G, R, -1).cpu().numpy().view(np.uint16), rqc)
    np.testing.assert_array_equal(f["kc"].view(G, R, -1).cpu().numpy().view(np.uint16), rkc)
    np.testing.assert_array_equal(f["qp"].view(G, -1).cpu().numpy(), rqp.reshape(G, -1))
    np.testing.assert_array_equal(f["kp"].view(G, -1).cpu().numpy(), rkp.reshape(G, -1))
    o = ref.forward(p, q, k, v, ps, pl, lamh, gsh, glh)
    rg = ref.backward(p, q, k, v, do, ps, pl, lamh, gsh, glh)

    def cpu(t, shape):
        return t.float().reshape(shape).cpu().numpy()

    errs = {n: rel_err(cpu(f[n], o[n].shape), o[n]) for n in ("O", "O_s", "O_lr", "lse", "d_lr")}
    errs["lse_elem_abs"] = lse_abs_err(cpu(f["lse"], o["lse"].shape), o["lse"])
    errs["d_lr_elem_rel"] = elem_rel_err(cpu(f["d_lr"], o["d_lr"].shape), o["d_lr"])
    for n in ("dQ", "dK", "dV", "dg_s", "dg_lr"):
        errs[n] = rel_err(cpu(g[n], rg[n].shape), rg[n])
    dl = np.zeros(w.H)
    for (b, h), x in zip(heads, rg["dlambda"]):
        dl[h] += x
    errs["dlambda"] = rel_err(g["dlambda"].cpu().numpy(), dl)
    print(f"[gpu rounds] {case} errors {errs}", flush=True)
    tol = TOL[w.dtype]
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{case}: errors above {tol}: {bad}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_repeated_round_adds_nothing(causal, dtype):
    """Hashing twice with the same hyperplanes gives the second round the same
    blocks as the first, so every pair it proposes is already held and its
    partials are empty: lse (a pair counted twice would raise it by about that
    pair's attention weight) matches the one-round call's to fp32 rounding, and so
    do the outputs and gradients. The several-round kernels are separate compiled
    variants whose fp32 results may differ from the one-round kernels' in the last
    bit; in bf16, where partial outputs and gradients are stored in bf16 between
    kernels, such a bit can flip one bf16 ulp (2^-8 relative), so the bf16 bar
    allows two."""
    w = wl("c", 1, 2, 512, 64, dtype, causal, 64, 64, "clusters", chunk=128, n_clusters=8,
           sigma=0.5)
    seed = 4200 + int(causal)
    print(f"[gpu rounds] repeated round causal={causal} {w}", flush=True)
    inp = W.gen_inputs(w, seed)
    lam = W.gen_lambda(w, seed, random=True)
    gs, glr = W.gen_gates(w, seed)
    f1, g1 = _run_gpu(w, inp, 1, lam, gs, glr)
    inp2 = dict(inp)
    inp2["planes_s"] = torch.stack([inp["planes_s"], inp["planes_s"]], dim=1).contiguous()
    f2, g2 = _run_gpu(w, inp2, 2, lam, gs, glr)
    P = f1["qp"].shape[-1]
    assert torch.equal(f2["qp"][..., :P], f1["qp"]) and torch.equal(f2["qp"][..., P:], f1["qp"])
    assert torch.equal(f2["kp"][..., :P], f1["kp"]) and torch.equal(f2["kp"][..., P:], f1["kp"])
    errs = {"lse_elem_abs": lse_abs_err(f2["lse"].cpu().numpy(), f1["lse"].cpu().numpy())}
    for n in ("O", "O_s", "O_lr", "d_lr"):
        errs[n] = rel_err(f2[n].float().cpu().numpy(), f1[n].float().cpu().numpy())
    for n in ("dQ", "dK", "dV", "dg_s", "dg_lr", "dlambda"):
        errs[n] = rel_err(g2[n].float().cpu().numpy(), g1[n].float().cpu().numpy())
    print(f"[gpu rounds] repeated round causal={causal} {dtype} differences {errs}", flush=True)
    tol = {"f32": 1e-5, "bf16": 2.0 ** -7}[dtype]
    # (lse: a few fp32 ulps at |lse| < 16)
    bad = {n: e for n, e in errs.items() if not e <= (8e-6 if n == "lse_elem_abs" else tol)}
    assert not bad, f"the repeated round changed the result: {bad}"
