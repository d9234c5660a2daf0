"""GPU parity of the forward path (elsaa_select, elsaa_lowrank_summary,
elsaa_fwd through the C ABI) against the oracle: selections bit-exact, summaries
and outputs within 1e-4 (fp32) / 2e-2 (bf16) max-relative error."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from parity_util import (CASES, TOL, all_heads, elem_rel_err, gpu_forward, head_arrays,
                         lse_abs_err, rel_err, wl)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("case", list(CASES))
def test_forward_parity(case):
    w, rand_lam, gates = CASES[case]
    seed = 1000 + len(case)
    print(f"[gpu fwd] {case} {w}", flush=True)
    inp = W.gen_inputs(w, seed)
    lam = W.gen_lambda(w, seed, random=rand_lam)
    gs, glr = W.gen_gates(w, seed) if gates else (None, None)
    cfg, _, g, _ = gpu_forward(w, inp, lam, gs, glr)
    heads = all_heads(w)
    q, k, v, _, ps, pl = head_arrays(w, inp, heads)
    p = ref.RefParams.from_workload(w)
    lamh = np.array([float(lam[h]) for _, h in heads])
    gsh = None if gs is None else np.stack([gs[b, h].double().numpy() for b, h in heads])
    glh = None if glr is None else np.stack([glr[b, h].double().numpy() for b, h in heads])
    qc, kc, qp, kp = ref.select(p, q, k, ps)
    A, z = ref.lowrank_summary(p, k, v, pl)
    o = ref.forward(p, q, k, v, ps, pl, lamh, gsh, glh)
    tol = TOL[w.dtype]
    G = len(heads)
    np.testing.assert_array_equal(g["qc"].view(G, -1).cpu().numpy().astype(np.uint16), qc)
    np.testing.assert_array_equal(g["kc"].view(G, -1).cpu().numpy().astype(np.uint16), kc)
    np.testing.assert_array_equal(g["qp"].view(G, -1).cpu().numpy(), qp.reshape(G, -1))
    np.testing.assert_array_equal(g["kp"].view(G, -1).cpu().numpy(), kp.reshape(G, -1))
    gA = g["A"].view(G, -1, w.d, w.r).transpose(-1, -2).cpu().numpy()
    gz = g["z"].view(G, -1, w.r).cpu().numpy()
    errs = {
        "A": rel_err(gA, A.reshape(G, -1, w.r, w.d)),
        "z": rel_err(gz, z.reshape(G, -1, w.r)),
    }
    for name, key in (("O", "O"), ("O_s", "O_s"), ("O_lr", "O_lr"), ("lse", "lse"),
                      ("d_lr", "d_lr")):
        errs[name] = rel_err(g[key].float().view(o[key].shape).cpu().numpy(), o[key])
    errs["lse_elem_abs"] = lse_abs_err(g["lse"].view(o["lse"].shape).cpu().numpy(), o["lse"])
    errs["d_lr_elem_rel"] = elem_rel_err(g["d_lr"].view(o["d_lr"].shape).cpu().numpy(), o["d_lr"])
    print(f"[gpu fwd] {case} errors {errs}", flush=True)
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, f"{case}: errors above {tol}: {bad}"


# Wider codes than the workloads use (9 to 12 hyperplanes: the hash kernel's
# two-threads-per-row split and the counting sort with up to 4096 bins, staged in
# LDS or not), causal and non-causal: codes and orders bit-exact.
SELECT_CASES = {
    "bits12_causal_f32_N65536_s16": wl("s", 1, 1, 65536, 32, "f32", True, 16, 16),
    "bits9_causal_bf16_N32768_s64": wl("s", 1, 2, 32768, 128, "bf16", True, 64, 16),
    "bits11_noncausal_bf16_N32768_s16": wl("s", 1, 1, 32768, 64, "bf16", False, 16, 16),
}


@pytest.mark.parametrize("case", list(SELECT_CASES))
def test_select_wide_codes(case):
    import sparse_rank_approximation_amd as S
    from parity_util import cfg_of, to_dev
    w = SELECT_CASES[case]
    print(f"[gpu select] {case} {w} bits {w.hash_bits}", flush=True)
    inp = W.gen_inputs(w, 4242)
    d = to_dev({k: inp[k] for k in ("q", "k", "planes_s")})
    qc, kc, qp, kp = S.select(cfg_of(w), d["q"], d["k"], d["planes_s"])
    torch.cuda.synchronize()
    heads = all_heads(w)
    q, k, _, _, ps, _ = head_arrays(w, inp, heads)
    rqc, rkc, rqp, rkp = ref.select(ref.RefParams.from_workload(w), q, k, ps)
    G = len(heads)
    np.testing.assert_array_equal(qc.view(G, -1).cpu().numpy().astype(np.uint16), rqc)
    np.testing.assert_array_equal(kc.view(G, -1).cpu().numpy().astype(np.uint16), rkc)
    np.testing.assert_array_equal(qp.view(G, -1).cpu().numpy(), rqp.reshape(G, -1))
    np.testing.assert_array_equal(kp.view(G, -1).cpu().numpy(), rkp.reshape(G, -1))


def test_forward_deterministic():
    w = CASES["causal_bf16_N1024_d128_s128"][0]
    inp = W.gen_inputs(w, 7)
    lam = W.gen_lambda(w, 7)
    _, _, g1, _ = gpu_forward(w, inp, lam)
    _, _, g2, _ = gpu_forward(w, inp, lam)
    for k in ("O", "O_s", "O_lr", "lse", "d_lr", "A", "z"):
        assert torch.equal(g1[k], g2[k]), k


def test_empty_problem_is_a_noop():
    import sparse_rank_approximation_amd as S
    cfg = S.ElsaaConfig(0, 4, 256, 64, torch.bfloat16, True, 64, lr_tables=2)
    q = torch.empty(0, 4, 256, 64, dtype=torch.bfloat16, device="cuda")
    ps = torch.zeros(4, cfg.bits, 64, device="cuda")
    qc, kc, qp, kp = S.select(cfg, q, q, ps)
    assert qc.numel() == 0 and qp.numel() == 0
