"""GPU parity of the learnable gate path (elsaa_gates_fwd / elsaa_gates_bwd through
the C ABI) composed with the operator: gates from the query's projection, the
forward and backward with those gates, and the gate path's gradient (dQ added in
place, dW, db), against the oracle's composition; plus the autograd Function with
a learned gate projection against the explicit calls."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from parity_util import TOL, all_heads, cfg_of, head_arrays, rel_err, to_dev, wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

CASES = {
    "gated_causal_bf16_N1024_d128": wl("g", 2, 2, 1024, 128, "bf16", True, 128, 128, "clusters",
                                       chunk=512, n_clusters=16, sigma=0.5),
    "gated_noncausal_f32_N512_d64": wl("g", 1, 3, 512, 64, "f32", False, 32, 32),
    "gated_causal_f32_ragged_d32": wl("g", 1, 2, 256, 32, "f32", True, 16, 48, chunk=32),
}


def gate_params(w, seed):
    g = torch.Generator().manual_seed(seed)
    return 0.2 * torch.randn(w.H, 2, w.d, generator=g), 0.5 * torch.randn(w.H, 2, generator=g)


def run_gpu(w, inp, Wg, bg, lam, fused=False):
    """The gated operator by explicit calls; fused: the forward as elsaa_fwd_fused
    (what the autograd function runs for a non-causal single-round problem)."""
    import sparse_rank_approximation_amd as S
    cfg = cfg_of(w)
    d = to_dev(inp)
    Wd, bd, lamd = Wg.cuda(), bg.cuda(), lam.cuda()
    gs, gl = S.gates(cfg, d["q"], Wd, bd)
    if fused:
        o = S.forward_fused(cfg, d["q"], d["k"], d["v"], d["planes_s"], d["planes_lr"], lamd, gs,
                            gl)
        qp, kp, A, z = o["q_perm"], o["k_perm"], o["A"], o["z"]
    else:
        _, _, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
        A, z = S.lowrank_summary(cfg, d["k"], d["v"], d["planes_lr"])
        o = S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lamd, gs, gl)
    g = S.backward(cfg, d["q"], d["k"], d["v"], d["do"], o["O_s"], o["O_lr"], d["planes_lr"], qp,
                   kp, A, z, o["lse"], o["d_lr"], lamd, gs, gl)
    dW, db = S.gates_backward(cfg, d["q"], Wd, gs, gl, g["dg_s"], g["dg_lr"], g["dQ"])
    torch.cuda.synchronize()
    return dict(g_s=gs, g_lr=gl, O=o["O"], dQ=g["dQ"], dK=g["dK"], dV=g["dV"], dW=dW, db=db,
                dlambda=g["dlambda"])


@pytest.mark.parametrize("case", list(CASES))
def test_gated_parity(case):
    w = CASES[case]
    seed = 5000 + len(case)
    print(f"[gpu gates] {case} {w}", flush=True)
    inp = W.gen_inputs(w, seed)
    Wg, bg = gate_params(w, seed)
    lam = W.gen_lambda(w, seed, random=True)
    got = run_gpu(w, inp, Wg, bg, lam)

    heads = all_heads(w)
    G = len(heads)
    q, k, v, do, ps, pl = head_arrays(w, inp, heads)
    p = ref.RefParams.from_workload(w)
    Wh = np.stack([Wg[h].double().numpy() for _, h in heads])
    bh = np.stack([bg[h].double().numpy() for _, h in heads])
    lamh = np.array([float(lam[h]) for _, h in heads])
    rgs, rgl = ref.gates_fwd(p, q, Wh, bh)
    o = ref.forward(p, q, k, v, ps, pl, lamh, rgs, rgl)
    rg = ref.backward(p, q, k, v, do, ps, pl, lamh, rgs, rgl)
    dq_gate, rdW, rdb = ref.gates_bwd(p, q, Wh, bh, rg["dg_s"], rg["dg_lr"])
    dW_h = np.zeros((w.H, 2, w.d))
    db_h = np.zeros((w.H, 2))
    for (b, h), x, y in zip(heads, rdW, rdb):
        dW_h[h] += x
        db_h[h] += y

    def cpu(t, shape):
        return t.float().reshape(shape).cpu().numpy()

    errs = {
        "g_s": rel_err(cpu(got["g_s"], rgs.shape), rgs),
        "g_lr": rel_err(cpu(got["g_lr"], rgl.shape), rgl),
        "O": rel_err(cpu(got["O"], o["O"].shape), o["O"]),
        "dQ": rel_err(cpu(got["dQ"], rg["dQ"].shape), rg["dQ"] + dq_gate),
        "dK": rel_err(cpu(got["dK"], rg["dK"].shape), rg["dK"]),
        "dV": rel_err(cpu(got["dV"], rg["dV"].shape), rg["dV"]),
        "dW": rel_err(got["dW"].cpu().numpy(), dW_h),
        "db": rel_err(got["db"].cpu().numpy(), db_h),
    }
    print(f"[gpu gates] {case} errors {errs}", flush=True)
    tol = TOL[w.dtype]
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{case}: errors above {tol}: {bad}"


def test_autograd_with_learned_gates_matches_calls():
    import sparse_rank_approximation_amd as S
    w = CASES["gated_noncausal_f32_N512_d64"]
    inp = W.gen_inputs(w, 17)
    Wg, bg = gate_params(w, 17)
    lam = torch.full((w.H,), 0.6)
    d = to_dev(inp)
    q = d["q"].clone().requires_grad_(True)
    k = d["k"].clone().requires_grad_(True)
    v = d["v"].clone().requires_grad_(True)
    gw = Wg.cuda().requires_grad_(True)
    gb = bg.cuda().requires_grad_(True)
    out = S.elsaa_attention(q, k, v, causal=False, block=w.block, lr_tables=w.lr_tables,
                            lam=lam.cuda(), planes_s=d["planes_s"], planes_lr=d["planes_lr"],
                            chunk=w.chunk, gate_w=gw, gate_b=gb)
    (out * d["do"]).sum().backward()
    assert not w.causal  # the autograd function takes the one-launch forward here
    got = run_gpu(w, inp, Wg, bg, lam, fused=True)
    assert torch.equal(out.detach(), got["O"])
    for name, t in (("dQ", q), ("dK", k), ("dV", v)):
        assert torch.equal(t.grad, got[name]), name
    assert torch.equal(gw.grad, got["dW"]) and torch.equal(gb.grad, got["db"])
