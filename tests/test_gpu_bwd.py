"""GPU parity of the backward (elsaa_bwd through the C ABI) against the oracle's
backward on the same seeded inputs: dQ, dK, dV, dlambda and the gate gradients
within 1e-4 (fp32) / 2e-2 (bf16) max-relative error; plus the autograd Function
and run-to-run determinism."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from parity_util import CASES, TOL, all_heads, gpu_forward, head_arrays, rel_err

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)


def gpu_backward(w, inp, lam, gs=None, glr=None):
    import sparse_rank_approximation_amd as S
    cfg, d, f, (lam_d, gs_d, glr_d) = gpu_forward(w, inp, lam, gs, glr)
    g = S.backward(cfg, d["q"], d["k"], d["v"], d["do"], f["O_s"], f["O_lr"], d["planes_lr"],
                   f["qp"], f["kp"], f["A"], f["z"], f["lse"], f["d_lr"], lam_d, gs_d, glr_d)
    torch.cuda.synchronize()
    return g


def oracle_backward(w, inp, lam, gs, glr):
    heads = all_heads(w)
    q, k, v, do, ps, pl = head_arrays(w, inp, heads)
    p = ref.RefParams.from_workload(w)
    lamh = np.array([float(lam[h]) for _, h in heads])
    gsh = None if gs is None else np.stack([gs[b, h].double().numpy() for b, h in heads])
    glh = None if glr is None else np.stack([glr[b, h].double().numpy() for b, h in heads])
    o = ref.backward(p, q, k, v, do, ps, pl, lamh, gsh, glh)
    dl = np.zeros(w.H)
    for (b, h), x in zip(heads, o["dlambda"]):
        dl[h] += x
    o["dlambda_h"] = dl
    return o


@pytest.mark.parametrize("case", list(CASES))
def test_backward_parity(case):
    w, rand_lam, gates = CASES[case]
    seed = 2000 + len(case)
    print(f"[gpu bwd] {case} {w}", flush=True)
    inp = W.gen_inputs(w, seed)
    lam = W.gen_lambda(w, seed, random=rand_lam)
    gs, glr = W.gen_gates(w, seed) if gates else (None, None)
    g = gpu_backward(w, inp, lam, gs, glr)
    o = oracle_backward(w, inp, lam, gs, glr)
    G = w.B * w.H
    errs = {}
    for name in ("dQ", "dK", "dV"):
        errs[name] = rel_err(g[name].float().view(G, w.N, w.d).cpu().numpy(), o[name])
    errs["dg_s"] = rel_err(g["dg_s"].view(G, w.N).cpu().numpy(), o["dg_s"])
    errs["dg_lr"] = rel_err(g["dg_lr"].view(G, w.N).cpu().numpy(), o["dg_lr"])
    errs["dlambda"] = rel_err(g["dlambda"].cpu().numpy(), o["dlambda_h"])
    print(f"[gpu bwd] {case} errors {errs}", flush=True)
    tol = TOL[w.dtype]
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, f"{case}: errors above {tol}: {bad}"


def test_backward_deterministic():
    w = CASES["causal_bf16_N1024_d128_s128"][0]
    inp = W.gen_inputs(w, 11)
    lam = W.gen_lambda(w, 11, random=True)
    g1 = gpu_backward(w, inp, lam)
    g2 = gpu_backward(w, inp, lam)
    for k in ("dQ", "dK", "dV", "dlambda", "dg_s", "dg_lr"):
        assert torch.equal(g1[k], g2[k]), k


def test_autograd_function_matches_calls():
    import sparse_rank_approximation_amd as S
    w = CASES["causal_f32_N512_d64_s32"][0]
    inp = W.gen_inputs(w, 13)
    d = {k: v.cuda() for k, v in inp.items()}
    lam = torch.full((w.H,), 0.7, device="cuda", requires_grad=True)
    q = d["q"].clone().requires_grad_(True)
    k = d["k"].clone().requires_grad_(True)
    v = d["v"].clone().requires_grad_(True)
    out = S.elsaa_attention(q, k, v, causal=True, block=w.block, lr_tables=w.lr_tables, lam=lam,
                            planes_s=d["planes_s"], planes_lr=d["planes_lr"], chunk=w.chunk)
    (out * d["do"]).sum().backward()
    g = gpu_backward(w, inp, torch.full((w.H,), 0.7))
    for name, t in (("dQ", q), ("dK", k), ("dV", v)):
        assert torch.equal(t.grad, g[name]), name
    assert torch.equal(lam.grad, g["dlambda"])
