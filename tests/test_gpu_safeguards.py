"""GPU tests of the debug safeguards and of how non-finite inputs travel.

- elsaa_check_orders accepts every order elsaa_select writes (causal and not,
  several rounds, a single causal block with no order at all), and counts exactly
  the violations planted in copies of them: an entry out of range, two entries
  swapped across segments, a repeated entry. The corrupted orders only ever reach
  the checker, which bounds-checks every entry before using it.
- With ELSAA_CHECK_ORDERS=1, elsaa_fwd refuses orders holding a repeated entry (an
  in-range corruption) before launching anything, and with valid orders gives the
  same bits as without the check.
- With ELSAA_CHECK_FINITE=1, elsaa_fwd / elsaa_bwd refuse inputs holding NaN or
  infinite entries and name the tensor.
- Without the flag, a NaN in V at key j0 (causal) makes every row i >= j0 of its
  head non-finite (the low-rank prefix sums include j0 from there on) and leaves
  the rows before the 128-token step holding j0, and every other head, finite (rows
  of that step before j0 may turn NaN too: a causally masked product multiplies
  the NaN by a zero weight); an infinite query row spoils only its own output; the
  backward runs to completion on such inputs."""
from __future__ import annotations

import pytest
import torch

import workloads as W
from parity_util import cfg_of, to_dev, wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)


def _select(w, R=1, seed=4500):
    import sparse_rank_approximation_amd as S
    inp = W.gen_inputs(w, seed)
    if R > 1:
        inp["planes_s"] = W.gen_planes_rounds(w, seed, R)
    cfg = cfg_of(w, hash_rounds=R)
    d = to_dev(inp)
    _, _, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    return cfg, d, qp, kp


@pytest.mark.parametrize("causal,R,N,s", [(True, 1, 1024, 64), (True, 2, 512, 32),
                                          (False, 2, 512, 64), (True, 1, 64, 64)])
def test_check_orders_accepts_selected_orders(causal, R, N, s):
    import sparse_rank_approximation_amd as S
    w = wl("c", 2, 2, N, 64, "bf16", causal, s, 64, chunk=64)
    print(f"[gpu safeguards] valid orders causal={causal} R={R} N={N} s={s}", flush=True)
    cfg, d, qp, kp = _select(w, R)
    bad = S.check_orders(cfg, qp, kp)
    torch.cuda.synchronize()
    assert bad.shape == (2, 2) and int(bad.abs().sum()) == 0, bad


def test_check_orders_counts_planted_violations():
    import sparse_rank_approximation_amd as S
    N, s = 1024, 64
    w = wl("c", 2, 2, N, 64, "bf16", True, s, 64, chunk=64)
    print(f"[gpu safeguards] planted violations {w}", flush=True)
    cfg, d, qp, kp = _select(w)
    bq, bk = qp.clone(), kp.clone()
    # head (0, 1): a query entry out of range -> the entry, and its token missing
    bq[0, 1, 5] = N + 7
    # head (1, 0): level 1 has two segments of 512; swap a query entry of each ->
    # two entries outside their half, and two tokens missing
    a, b = N // 2 + 3, N // 2 + N // 4 + 9
    bq[1, 0, a], bq[1, 0, b] = qp[1, 0, b], qp[1, 0, a]
    # head (1, 1): a key entry repeated within its half -> one token twice, one missing
    bk[1, 1, 11] = kp[1, 1, 10]
    bad = S.check_orders(cfg, bq, bk).cpu()
    torch.cuda.synchronize()
    assert bad.tolist() == [[0, 2], [4, 2]], bad


def test_env_check_orders_refuses_bad_orders(monkeypatch):
    import sparse_rank_approximation_amd as S
    from sparse_rank_approximation_amd import _lib
    w = wl("c", 1, 2, 512, 64, "bf16", True, 64, 64, chunk=128)
    print(f"[gpu safeguards] ELSAA_CHECK_ORDERS {w}", flush=True)
    cfg, d, qp, kp = _select(w)
    A, z = S.lowrank_summary(cfg, d["k"], d["v"], d["planes_lr"])
    lam = torch.ones(w.H, device="cuda")
    ref = S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lam)
    monkeypatch.setenv("ELSAA_CHECK_ORDERS", "1")
    got = S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lam)
    torch.cuda.synchronize()
    for n in ("O", "O_s", "lse"):
        assert torch.equal(got[n], ref[n]), n
    bk = kp.clone()
    bk[0, 1, 100] = kp[0, 1, 101]  # in range: a repeated key
    with pytest.raises(_lib.ElsaaError, match="head 1"):
        S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, bk, A, z, lam)
    torch.cuda.synchronize()


def _forward_backward(w, inp, cfg):
    import sparse_rank_approximation_amd as S
    d = to_dev(inp)
    _, _, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    A, z = S.lowrank_summary(cfg, d["k"], d["v"], d["planes_lr"])
    lam = torch.ones(w.H, device="cuda")
    f = S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lam)
    g = S.backward(cfg, d["q"], d["k"], d["v"], d["do"], f["O_s"], f["O_lr"], d["planes_lr"], qp,
                   kp, A, z, f["lse"], f["d_lr"], lam)
    torch.cuda.synchronize()
    return f, g


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nonfinite_inputs_propagate_where_they_should(dtype):
    w = wl("c", 1, 2, 512, 64, dtype, True, 64, 64, chunk=128)
    j0, i0 = 300, 123
    print(f"[gpu safeguards] NaN/Inf propagation {w}", flush=True)
    inp = W.gen_inputs(w, 4600)
    inp["v"][0, 1, j0, 7] = float("nan")
    inp["q"][0, 0, i0, 3] = float("inf")
    cfg = cfg_of(w)
    f, g = _forward_backward(w, inp, cfg)
    O = f["O"].float().cpu()
    fin = torch.isfinite(O).all(dim=-1)[0]  # [H, N]
    step0 = (j0 // 128) * 128
    assert bool(fin[1, :step0].all()) and not bool(fin[1, j0:].any())
    assert not bool(fin[0, i0]) and bool(fin[0, :i0].all()) and bool(fin[0, i0 + 1:].all())
    for n in ("dQ", "dK", "dV"):
        assert g[n].shape == O.shape


def test_env_check_finite_names_the_tensor(monkeypatch):
    import sparse_rank_approximation_amd as S
    from sparse_rank_approximation_amd import _lib
    w = wl("c", 1, 2, 256, 32, "f32", True, 32, 32, chunk=64)
    print(f"[gpu safeguards] ELSAA_CHECK_FINITE {w}", flush=True)
    inp = W.gen_inputs(w, 4700)
    cfg = cfg_of(w)
    monkeypatch.setenv("ELSAA_CHECK_FINITE", "1")
    f, g = _forward_backward(w, inp, cfg)  # clean inputs pass
    assert bool(torch.isfinite(f["O"]).all())
    inp["v"][0, 1, 17, 0] = float("inf")
    d = to_dev(inp)
    _, _, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
    A, z = S.lowrank_summary(cfg, d["k"], d["v"], d["planes_lr"])
    lam = torch.ones(w.H, device="cuda")
    with pytest.raises(_lib.ElsaaError, match="V holds 1 NaN"):
        S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lam)
    torch.cuda.synchronize()
