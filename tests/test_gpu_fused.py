"""GPU parity of the fused non-causal forward (elsaa_fwd_fused through the C ABI)
against the oracle on the same seeded inputs: codes and orders bit for bit (and
the same as elsaa_select's), A and z, the outputs and the saved statistics within
1e-4 (fp32) / 2e-2 (bf16) max-relative error; the backward taken from its saved
tensors against the oracle's backward; run-to-run determinism; and the full-size
vision workload (B64 H12 N1024 d64) in the launch configuration bench.py times, on
sampled heads; and codes of rows on or near their hyperplanes (the products cannot
decide those bits, the fp64 chain does) bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from parity_util import (CASES, TOL, all_heads, cfg_of, elem_rel_err, head_arrays, lse_abs_err,
                         rel_err, to_dev, wl)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

# (workload, random lambda, gates): every head dimension, block sizes 16 to 128
# (one to four waves per block, blocks of 16 padded to a 32-row tile), padded
# table counts 2, 4 and 8, ragged N, both dtypes.
FUSED_CASES = {
    "tiny_f32": CASES["tiny_f32"],
    "vit_bf16_N1024_d64_s32": CASES["vit_bf16_N1024_d64_s32"],
    "ragged_noncausal_f32_N96": CASES["ragged_noncausal_f32_N96"],
    "bf16_N2048_d128_s128_r128": (wl("f", 1, 2, 2048, 128, "bf16", False, 128, 128, "clusters",
                                     n_clusters=16, sigma=0.5), True, True),
    "bf16_N512_d32_s64_r64": (wl("f", 2, 1, 512, 32, "bf16", False, 64, 64), True, False),
    "f32_N512_d64_s16_r48": (wl("f", 1, 2, 512, 64, "f32", False, 16, 48), False, True),
    "bf16_N4160_d64_s32_bits7": (wl("f", 1, 1, 4160, 64, "bf16", False, 32, 32, "clusters",
                                    n_clusters=64, sigma=0.3), True, True),
}


def fused_forward(w, inp, lam, gs=None, glr=None):
    import sparse_rank_approximation_amd as S
    cfg = cfg_of(w)
    d = to_dev(inp)
    lam_d = lam.to("cuda", torch.float32)
    gs_d = None if gs is None else gs.to("cuda", torch.float32).contiguous()
    glr_d = None if glr is None else glr.to("cuda", torch.float32).contiguous()
    out = S.forward_fused(cfg, d["q"], d["k"], d["v"], d["planes_s"], d["planes_lr"], lam_d, gs_d,
                          glr_d)
    torch.cuda.synchronize()
    return cfg, d, out, (lam_d, gs_d, glr_d)


def oracle_inputs(w, inp, lam, gs, glr, heads):
    q, k, v, do, ps, pl = head_arrays(w, inp, heads)
    lamh = np.array([float(lam[h]) for _, h in heads])
    gsh = None if gs is None else np.stack([gs[b, h].double().numpy() for b, h in heads])
    glh = None if glr is None else np.stack([glr[b, h].double().numpy() for b, h in heads])
    return q, k, v, do, ps, pl, lamh, gsh, glh


@pytest.mark.parametrize("case", list(FUSED_CASES))
def test_fused_forward_parity(case):
    w, rand_lam, gates = FUSED_CASES[case]
    seed = 3000 + len(case)
    print(f"[gpu fused] {case} {w}", flush=True)
    inp = W.gen_inputs(w, seed)
    lam = W.gen_lambda(w, seed, random=rand_lam)
    gs, glr = W.gen_gates(w, seed) if gates else (None, None)
    cfg, d, g, _ = fused_forward(w, inp, lam, gs, glr)
    heads = all_heads(w)
    q, k, v, _, ps, pl, lamh, gsh, glh = oracle_inputs(w, inp, lam, gs, glr, heads)
    p = ref.RefParams.from_workload(w)
    qc, kc, qp, kp = ref.select(p, q, k, ps)
    A, z = ref.lowrank_summary(p, k, v, pl)
    o = ref.forward(p, q, k, v, ps, pl, lamh, gsh, glh)
    G = len(heads)
    np.testing.assert_array_equal(g["q_code"].view(G, -1).cpu().numpy().astype(np.uint16), qc)
    np.testing.assert_array_equal(g["k_code"].view(G, -1).cpu().numpy().astype(np.uint16), kc)
    np.testing.assert_array_equal(g["q_perm"].view(G, -1).cpu().numpy(), qp.reshape(G, -1))
    np.testing.assert_array_equal(g["k_perm"].view(G, -1).cpu().numpy(), kp.reshape(G, -1))
    gA = g["A"].view(G, -1, w.d, w.r).transpose(-1, -2).cpu().numpy()
    errs = {"A": rel_err(gA, A.reshape(G, -1, w.r, w.d)),
            "z": rel_err(g["z"].view(G, -1, w.r).cpu().numpy(), z.reshape(G, -1, w.r))}
    for name in ("O", "O_s", "O_lr", "lse", "d_lr"):
        errs[name] = rel_err(g[name].float().view(o[name].shape).cpu().numpy(), o[name])
    errs["lse_elem_abs"] = lse_abs_err(g["lse"].view(o["lse"].shape).cpu().numpy(), o["lse"])
    errs["d_lr_elem_rel"] = elem_rel_err(g["d_lr"].view(o["d_lr"].shape).cpu().numpy(), o["d_lr"])
    print(f"[gpu fused] {case} errors {errs}", flush=True)
    tol = TOL[w.dtype]
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{case}: errors above {tol}: {bad}"


@pytest.mark.parametrize("case", ["vit_bf16_N1024_d64_s32", "f32_N512_d64_s16_r48",
                                  "bf16_N2048_d128_s128_r128"])
def test_backward_from_fused_forward(case):
    """elsaa_bwd on what the fused forward saved: gradients within the bar of the
    oracle's backward."""
    import sparse_rank_approximation_amd as S
    w, rand_lam, gates = FUSED_CASES[case]
    seed = 4000 + len(case)
    inp = W.gen_inputs(w, seed)
    lam = W.gen_lambda(w, seed, random=rand_lam)
    gs, glr = W.gen_gates(w, seed) if gates else (None, None)
    cfg, d, f, (lam_d, gs_d, glr_d) = fused_forward(w, inp, lam, gs, glr)
    g = S.backward(cfg, d["q"], d["k"], d["v"], d["do"], f["O_s"], f["O_lr"], d["planes_lr"],
                   f["q_perm"], f["k_perm"], f["A"], f["z"], f["lse"], f["d_lr"], lam_d, gs_d,
                   glr_d)
    torch.cuda.synchronize()
    heads = all_heads(w)
    q, k, v, do, ps, pl, lamh, gsh, glh = oracle_inputs(w, inp, lam, gs, glr, heads)
    o = ref.backward(ref.RefParams.from_workload(w), q, k, v, do, ps, pl, lamh, gsh, glh)
    G = len(heads)
    errs = {n: rel_err(g[n].float().view(G, w.N, w.d).cpu().numpy(), o[n]) for n in ("dQ", "dK", "dV")}
    errs["dg_s"] = rel_err(g["dg_s"].view(G, w.N).cpu().numpy(), o["dg_s"])
    errs["dg_lr"] = rel_err(g["dg_lr"].view(G, w.N).cpu().numpy(), o["dg_lr"])
    dl = np.zeros(w.H)
    for (b, h), x in zip(heads, o["dlambda"]):
        dl[h] += x
    errs["dlambda"] = rel_err(g["dlambda"].cpu().numpy(), dl)
    print(f"[gpu fused bwd] {case} errors {errs}", flush=True)
    tol = TOL[w.dtype]
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{case}: errors above {tol}: {bad}"


def test_fused_selection_equals_two_call_selection_and_is_deterministic():
    import sparse_rank_approximation_amd as S
    w = FUSED_CASES["bf16_N2048_d128_s128_r128"][0]
    inp = W.gen_inputs(w, 21)
    lam = W.gen_lambda(w, 21, random=True)
    cfg, d, f1, _ = fused_forward(w, inp, lam)
    _, _, f2, _ = fused_forward(w, inp, lam)
    for n in f1:
        assert torch.equal(f1[n], f2[n]), n
    qc, kc, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    torch.cuda.synchronize()
    for n, t in (("q_code", qc), ("k_code", kc), ("q_perm", qp), ("k_perm", kp)):
        assert torch.equal(f1[n], t), n


def test_fused_full_size_vision_workload():
    """B64 H12 N1024 d64 bf16 non-causal (the vision workload at full size):
    every head's orders equal elsaa_select's; sampled heads against the oracle."""
    import sparse_rank_approximation_amd as S
    cid = 5
    w = W.WORKLOADS[cid]
    inp = W.gen_inputs(w, W.workload_seed(cid))
    lam = torch.ones(w.H)
    cfg, d, f, _ = fused_forward(w, inp, lam)
    qc, kc, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    torch.cuda.synchronize()
    assert torch.equal(f["q_perm"], qp) and torch.equal(f["k_perm"], kp)
    heads = [(0, 0), (17, 6), (63, 11)]
    q, k, v, _, ps, pl, lamh, _, _ = oracle_inputs(w, inp, lam, None, None, heads)
    o = ref.forward(ref.RefParams.from_workload(w), q, k, v, ps, pl, lamh)

    def pick(t, shape):
        return np.stack([t[b, h].float().cpu().numpy() for b, h in heads]).reshape(shape)

    errs = {n: rel_err(pick(f[n], o[n].shape), o[n]) for n in ("O", "O_s", "O_lr", "lse", "d_lr")}
    print(f"[gpu fused full] config {cid}: errors {errs}", flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL[w.dtype]}
    assert not bad, f"errors above {TOL[w.dtype]}: {bad}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_codes_on_and_near_hyperplanes(dtype):
    """Rows whose projections are exactly zero or within a few ulps of it,
    subnormal rows, a hyperplane of zeros and a hyperplane holding a value below
    2^-100: every code and order equal to the oracle's and to elsaa_select's."""
    import sparse_rank_approximation_amd as S
    w = wl("f", 1, 2, 512, 64, dtype, False, 32, 32)  # 4 hyperplanes per head
    inp = W.gen_inputs(w, 5150)
    q, k, ps = inp["q"].clone(), inp["k"].clone(), inp["planes_s"].clone()
    # Head 0: hyperplanes 0 and 3 pair each even coordinate with its negation, so
    # rows with x[2i] = x[2i + 1] lie exactly on them (every chain step cancels).
    for b in (0, 3):
        ps[0, b, 1::2] = -ps[0, b, 0::2]
    for x in (q, k):
        x[0, 0, 0:200, 1::2] = x[0, 0, 0:200, 0::2]
        # one pair off by an ulp: a projection a few ulps from zero
        x[0, 0, 100:200, 7] = x[0, 0, 100:200, 6] * (1 + 2.0 ** -7)
        # subnormal rows (products the unit flushes)
        x[0, 0, 300:310] = torch.where(x[0, 0, 300:310] > 0, 3e-39, -3e-39).to(x.dtype)
    # Head 1: a hyperplane of zeros and one holding a value below 2^-100.
    ps[1, 1] = 0.0
    ps[1, 2, 5] = 1e-35
    inp.update(q=q.contiguous(), k=k.contiguous(), planes_s=ps.contiguous())
    lam = torch.ones(w.H)
    cfg, d, f, _ = fused_forward(w, inp, lam)
    qc, kc, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    torch.cuda.synchronize()
    heads = all_heads(w)
    hq, hk, _, _, hps, _ = head_arrays(w, inp, heads)
    rqc, rkc, rqp, rkp = ref.select(ref.RefParams.from_workload(w), hq, hk, hps)
    G = len(heads)
    np.testing.assert_array_equal(f["q_code"].view(G, -1).cpu().numpy().astype(np.uint16), rqc)
    np.testing.assert_array_equal(f["k_code"].view(G, -1).cpu().numpy().astype(np.uint16), rkc)
    np.testing.assert_array_equal(f["q_perm"].view(G, -1).cpu().numpy(), rqp.reshape(G, -1))
    np.testing.assert_array_equal(f["k_perm"].view(G, -1).cpu().numpy(), rkp.reshape(G, -1))
    for n, t in (("q_code", qc), ("k_code", kc), ("q_perm", qp), ("k_perm", kp)):
        assert torch.equal(f[n], t), n
    # the planted rows did land on the hyperplanes: bit 0 clear on head 0's paired rows
    assert not (rqc[0, 0:100] & 1).any() and not (rqc[1] & (1 << 1)).any()
