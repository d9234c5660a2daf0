"""Pins of the oracle against what the ELSAA paper and plain mathematics fix:
exact-rational hash signs, the sort order the sortLSH description implies, the
closed-form causal support size, brute-force dense masked softmax, textbook
attention when the support is full, closed forms of the RACE branch, the
fusion's special cases, permutation invariance, finite differences and
autograd of a dense formulation. CPU only."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import dense_check as D
import workloads as W
from oracle import ref


def small(causal, N=128, d=16, block=16, r=32, lr_bits=4, gen="iid", dtype="f32", chunk=32,
          H=1, **ga):
    return W.Workload("t", 1, H, N, d, dtype, causal, block, r, gen, ga, lr_bits=lr_bits,
                      chunk=chunk)


def head(w, seed, h=0):
    q, k = W.gen_qk(w, seed, 0, h)
    dt = w.torch_dtype
    q, k = q.to(dt).double(), k.to(dt).double()
    v = W.gen_v(w, seed, 0, h).to(dt).double()
    do = W.gen_do(w, seed, 0, h).to(dt).double()
    ps, pl = W.gen_planes(w, seed)
    return q.numpy(), k.numpy(), v.numpy(), do.numpy(), ps[h:h + 1].numpy(), pl[h:h + 1].numpy()


def run_select(w, p, q, k, ps):
    return ref.select(p, q[None], k[None], ps)


# ----------------------------------------------------------------------------- selection

@pytest.mark.parametrize("causal", [False, True])
def test_hash_codes_equal_exact_rational_sign(causal):
    w = small(causal, N=64, d=24, block=8)
    p = ref.RefParams.from_workload(w)
    q, k, *_, ps, _ = head(w, 11)
    qc, kc, _, _ = run_select(w, p, q, k, ps)
    np.testing.assert_array_equal(qc[0], D.exact_sign_bits(q, ps[0]))
    np.testing.assert_array_equal(kc[0], D.exact_sign_bits(k, ps[0]))


def _check_sorted(perm, tokens, code, bits):
    rank = D.gray_rank_table(bits)[code.astype(np.int64)]
    assert sorted(perm.tolist()) == sorted(tokens)
    key = [(int(rank[t]), int(t)) for t in perm]
    assert key == sorted(key), "order must be by Gray rank, ties by ascending token index"


def test_noncausal_orders_sorted_by_gray_rank_then_index():
    w = small(False, N=256, d=16, block=16)
    p = ref.RefParams.from_workload(w)
    q, k, *_, ps, _ = head(w, 3)
    qc, kc, qp, kp = run_select(w, p, q, k, ps)
    assert qp.shape == (1, 1, 256)
    _check_sorted(qp[0, 0], range(256), qc[0], w.hash_bits)
    _check_sorted(kp[0, 0], range(256), kc[0], w.hash_bits)


def test_causal_orders_per_level_and_segment():
    w = small(True, N=256, d=16, block=16)
    p = ref.RefParams.from_workload(w)
    q, k, *_, ps, _ = head(w, 5)
    qc, kc, qp, kp = run_select(w, p, q, k, ps)
    assert qp.shape == (1, 4, 128)
    for lev in range(4):
        n = 256 >> lev
        for a in range(0, 256, n):
            off = (a // n) * (n // 2)
            _check_sorted(qp[0, lev, off:off + n // 2], range(a + n // 2, a + n), qc[0], w.hash_bits)
            _check_sorted(kp[0, lev, off:off + n // 2], range(a, a + n // 2), kc[0], w.hash_bits)


def test_gray_rank_table_is_a_gray_order():
    t = D.gray_rank_table(6)
    inv = np.argsort(t)
    for a, b in zip(inv[:-1], inv[1:]):
        assert bin(int(a) ^ int(b)).count("1") == 1


def test_causal_support_closed_form_and_causality():
    w = small(True, N=256, d=16, block=16)
    p = ref.RefParams.from_workload(w)
    q, k, *_, ps, _ = head(w, 7)
    _, _, qp, kp = run_select(w, p, q, k, ps)
    M = D.support_mask(256, 16, True, qp[0], kp[0])
    i = np.arange(256)
    expect = (i % 16) + 1 + 16 * np.array([D.popcount(x) for x in i // 16])
    np.testing.assert_array_equal(M.sum(1), expect)
    assert not np.triu(M, 1).any(), "no key after its query"


def test_noncausal_support_is_block_diagonal_after_permutation():
    w = small(False, N=128, d=16, block=16)
    p = ref.RefParams.from_workload(w)
    q, k, *_, ps, _ = head(w, 9)
    _, _, qp, kp = run_select(w, p, q, k, ps)
    M = D.support_mask(128, 16, False, qp[0], kp[0])
    assert (M.sum(1) == 16).all() and (M.sum(0) == 16).all()
    Mp = M[np.ix_(qp[0, 0], kp[0, 0])]
    blk = np.kron(np.eye(8, dtype=bool), np.ones((16, 16), bool))
    np.testing.assert_array_equal(Mp, blk)


# ----------------------------------------------------------------------------- sparse branch

@pytest.mark.parametrize("causal,gen", [(False, "iid"), (True, "iid"), (True, "clusters")])
def test_sparse_branch_equals_dense_masked_softmax(causal, gen):
    ga = dict(n_clusters=8, sigma=0.3) if gen == "clusters" else {}
    w = small(causal, N=256, d=16, block=16, gen=gen, **ga)
    p = ref.RefParams.from_workload(w)
    q, k, v, _, ps, pl = head(w, 21)
    _, _, qp, kp = run_select(w, p, q, k, ps)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.ones(1))
    M = D.support_mask(256, 16, causal, qp[0], kp[0])
    dn = D.dense_forward(*(torch.from_numpy(x) for x in (q, k, v)), M, torch.from_numpy(pl[0]), 1.0,
                         causal, 1 / math.sqrt(16))
    np.testing.assert_allclose(out["O_s"][0], dn["O_s"].numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["lse"][0], dn["lse"].numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_full_support_is_exact_attention(causal):
    w = small(causal, N=64, d=16, block=64)
    p = ref.RefParams.from_workload(w)
    q, k, v, _, ps, pl = head(w, 4)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.zeros(1), g_lr=np.zeros((1, 64)))
    S = q @ k.T / 4.0
    if causal:
        S = np.where(np.tril(np.ones((64, 64), bool)), S, -np.inf)
    mx = S.max(1, keepdims=True)
    e = np.exp(S - mx)
    Oex = (e @ v) / e.sum(1, keepdims=True)
    np.testing.assert_allclose(out["O_s"][0], Oex, atol=1e-12)
    np.testing.assert_allclose(out["lse"][0], (mx[:, 0] + np.log(e.sum(1))), atol=1e-12)
    # lambda = 0 with the default eps = 1e-6 gives m = d_s / (d_s + eps); with
    # g_lr = 0 the fused output is that multiple of exact attention.
    ds = np.exp(mx[:, 0]) * e.sum(1)
    np.testing.assert_allclose(out["O"][0], (ds / (ds + 1e-6))[:, None] * Oex, atol=1e-12)


def test_full_support_eps_zero_is_exactly_attention():
    w = small(False, N=64, d=16, block=64)
    p = ref.RefParams.from_workload(w, eps=0.0)
    q, k, v, _, ps, pl = head(w, 6)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.zeros(1), g_lr=np.zeros((1, 64)))
    S = q @ k.T / 4.0
    e = np.exp(S - S.max(1, keepdims=True))
    np.testing.assert_allclose(out["O"][0], (e @ v) / e.sum(1, keepdims=True), atol=1e-12)


# ----------------------------------------------------------------------------- low-rank branch

def test_features_normalised_and_product_of_sigmoids():
    w = small(False, d=16, r=48, lr_bits=4)
    p = ref.RefParams.from_workload(w, tau=0.7)
    q, *_, pl = head(w, 13)
    phi = ref.features(p, pl[0], q[:20])
    L, g = 3, 4
    np.testing.assert_allclose(phi.reshape(20, L, 16).sum(-1), 1.0, atol=1e-14)
    u = (1 / 4.0) * np.einsum("ltd,nd->nlt", pl[0].astype(np.float64), q[:20])
    sig = lambda x: 1 / (1 + np.exp(-x))
    prod = np.ones((20, L, 16))
    for b in range(16):
        for t in range(g):
            sgn = 1.0 if (b >> t) & 1 else -1.0
            prod[:, :, b] *= sig(2 * sgn * u[:, :, t] / 0.7)
    np.testing.assert_allclose(phi.reshape(20, L, 16), prod, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_lowrank_without_hyperplanes_is_uniform_mean(causal):
    w = small(causal, N=128, d=16, r=3, lr_bits=0)
    p = ref.RefParams.from_workload(w)
    q, k, v, _, ps, pl = head(w, 17)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.ones(1))
    n = np.arange(1, 129) if causal else np.full(128, 128)
    mean = np.cumsum(v, 0) / n[:, None] if causal else np.broadcast_to(v.mean(0), v.shape)
    np.testing.assert_allclose(out["O_lr"][0], mean, atol=1e-12)
    np.testing.assert_allclose(out["d_lr"][0], 3 * n, atol=1e-9)


def test_lowrank_large_tau_is_uniform_over_buckets():
    w = small(True, N=64, d=16, r=32, lr_bits=4)
    p = ref.RefParams.from_workload(w, tau=1e12)
    q, k, v, _, ps, pl = head(w, 19)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.ones(1))
    n = np.arange(1, 65)
    np.testing.assert_allclose(out["O_lr"][0], np.cumsum(v, 0) / n[:, None], atol=1e-9)
    np.testing.assert_allclose(out["d_lr"][0], 2 * n / 16.0, atol=1e-9)


@pytest.mark.parametrize("causal", [False, True])
def test_lowrank_equals_brute_force_double_sum(causal):
    w = small(causal, N=128, d=16, r=32)
    p = ref.RefParams.from_workload(w)
    q, k, v, _, ps, pl = head(w, 23)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.ones(1))
    fq = D.features_torch(torch.from_numpy(q), torch.from_numpy(pl[0]), 0.25, 1.0).numpy()
    fk = D.features_torch(torch.from_numpy(k), torch.from_numpy(pl[0]), 0.25, 1.0).numpy()
    num = np.zeros_like(v)
    den = np.zeros(128)
    for i in range(128):
        for j in range(128):
            if causal and j > i:
                continue
            wij = float(fq[i] @ fk[j])
            num[i] += wij * v[j]
            den[i] += wij
    np.testing.assert_allclose(out["d_lr"][0], den, rtol=1e-12)
    np.testing.assert_allclose(out["O_lr"][0], num / den[:, None], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_summary_statistics(causal):
    w = small(causal, N=128, d=16, r=32, chunk=32)
    p = ref.RefParams.from_workload(w)
    _, k, v, _, ps, pl = head(w, 29)
    A, z = ref.lowrank_summary(p, k[None], v[None], pl)
    fk = D.features_torch(torch.from_numpy(k), torch.from_numpy(pl[0]), 0.25, 1.0).numpy()
    if not causal:
        np.testing.assert_allclose(A[0], fk.T @ v, atol=1e-11)
        np.testing.assert_allclose(z[0].sum(), 2 * 128, rtol=1e-12)  # L = 2 tables
    else:
        assert A.shape == (1, 4, 32, 16)
        for c in range(4):
            np.testing.assert_allclose(A[0, c], fk[:32 * c].T @ v[:32 * c], atol=1e-11)
            np.testing.assert_allclose(z[0, c], fk[:32 * c].sum(0), atol=1e-12)


# ----------------------------------------------------------------------------- fusion

def test_fusion_with_unit_values():
    w = small(True, N=128, d=16)
    p = ref.RefParams.from_workload(w)
    q, k, _, _, ps, pl = head(w, 31)
    gs, gl = W.gen_gates(w, 31)
    v = np.ones((128, 16))
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.array([0.8]), gs[0].numpy(),
                      gl[0].numpy())
    np.testing.assert_allclose(out["O_s"][0], 1.0, atol=1e-12)
    np.testing.assert_allclose(out["O_lr"][0], 1.0, atol=1e-12)
    m = (out["O"][0, :, 0] - gl[0, 0].numpy()) / gs[0, 0].numpy()
    assert (m > 0).all() and (m < 1).all()
    ds = np.exp(out["lse"][0])
    np.testing.assert_allclose(m, ds / (ds + 0.8 * out["d_lr"][0] + 1e-6), rtol=1e-12)


def test_fusion_lambda_eps_zero_is_plain_sum():
    w = small(False, N=128, d=16)
    p = ref.RefParams.from_workload(w, eps=0.0)
    q, k, v, _, ps, pl = head(w, 37)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.zeros(1))
    np.testing.assert_allclose(out["O"][0], out["O_s"][0] + out["O_lr"][0], atol=1e-14)


def test_fusion_lambda_large_keeps_low_rank_only():
    w = small(False, N=128, d=16)
    p = ref.RefParams.from_workload(w)
    q, k, v, _, ps, pl = head(w, 41)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, np.array([1e14]))
    np.testing.assert_allclose(out["O"][0], out["O_lr"][0], atol=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_fused_weights_nonnegative_with_gate_row_sums(causal):
    w = small(causal, N=128, d=16)
    p = ref.RefParams.from_workload(w)
    q, k, v, _, ps, pl = head(w, 43)
    gs, gl = W.gen_gates(w, 43)
    lam = np.array([1.7])
    _, _, qp, kp = run_select(w, p, q, k, ps)
    out = ref.forward(p, q[None], k[None], v[None], ps, pl, lam, gs[0].numpy(), gl[0].numpy())
    M = D.support_mask(128, 16, causal, qp[0], kp[0])
    dn = D.dense_forward(*(torch.from_numpy(x) for x in (q, k, v)), M, torch.from_numpy(pl[0]), 1.7,
                         causal, 0.25, g_s=gs[0, 0].double(), g_lr=gl[0, 0].double())
    S = torch.from_numpy(q @ k.T * 0.25).masked_fill(~torch.from_numpy(M), float("-inf"))
    P = torch.softmax(S, 1).numpy()
    fq = D.features_torch(torch.from_numpy(q), torch.from_numpy(pl[0]), 0.25, 1.0).numpy()
    fk = D.features_torch(torch.from_numpy(k), torch.from_numpy(pl[0]), 0.25, 1.0).numpy()
    Kl = fq @ fk.T
    if causal:
        Kl = np.tril(Kl)
    Kl /= Kl.sum(1, keepdims=True)
    m = dn["m"].numpy()
    g1, g2 = gs[0, 0].numpy(), gl[0, 0].numpy()
    Wf = (g1 * m)[:, None] * P + g2[:, None] * Kl
    assert (Wf >= 0).all()
    np.testing.assert_allclose(Wf.sum(1), g1 * m + g2, atol=1e-12)
    np.testing.assert_allclose(out["O"][0], Wf @ v, atol=1e-11)


# ----------------------------------------------------------------------------- invariance

def test_noncausal_key_value_permutation():
    w = small(False, N=128, d=16)
    p = ref.RefParams.from_workload(w)
    q, k, v, _, ps, pl = head(w, 47)
    _, kc, _, _ = run_select(w, p, q, k, ps)
    base = ref.forward(p, q[None], k[None], v[None], ps, pl, np.ones(1))
    # Moving keys so that relative order inside each hash-rank class is kept leaves
    # every block, hence the output, unchanged.
    rank = D.gray_rank_table(w.hash_bits)[kc[0].astype(np.int64)]
    pi = np.argsort(-rank, kind="stable")
    out = ref.forward(p, q[None], k[pi][None], v[pi][None], ps, pl, np.ones(1))
    np.testing.assert_allclose(out["O"][0], base["O"][0], atol=1e-12)
    # The low-rank branch is invariant under any key/value permutation.
    pi = np.random.default_rng(0).permutation(128)
    out = ref.forward(p, q[None], k[pi][None], v[pi][None], ps, pl, np.ones(1))
    np.testing.assert_allclose(out["O_lr"][0], base["O_lr"][0], atol=1e-12)
    np.testing.assert_allclose(out["d_lr"][0], base["d_lr"][0], rtol=1e-12)


def test_heads_are_independent():
    w = small(True, N=128, d=16, H=2)
    p = ref.RefParams.from_workload(w)
    h0, h1 = head(w, 53, 0), head(w, 53, 1)
    both = ref.forward(p, np.stack([h0[0], h1[0]]), np.stack([h0[1], h1[1]]),
                       np.stack([h0[2], h1[2]]), np.concatenate([h0[4], h1[4]]),
                       np.concatenate([h0[5], h1[5]]), np.array([1.0, 2.0]))
    one = ref.forward(p, h1[0][None], h1[1][None], h1[2][None], h1[4], h1[5], np.array([2.0]))
    np.testing.assert_array_equal(both["O"][1], one["O"][0])


# ----------------------------------------------------------------------------- backward

def _loss(p, q, k, v, do, ps, pl, lam, gs, gl):
    o = ref.forward(p, q[None], k[None], v[None], ps, pl, np.array([lam]), gs[None], gl[None])
    return float((o["O"][0] * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    w = small(causal, N=64, d=8, block=8, r=32, chunk=16)
    p = ref.RefParams.from_workload(w)
    q, k, v, do, ps, pl = head(w, 59)
    gs, gl = (x[0, 0].numpy().astype(np.float64) for x in W.gen_gates(w, 59))
    lam = 0.9
    g = ref.backward(p, q[None], k[None], v[None], do[None], ps, pl, np.array([lam]), gs[None],
                     gl[None])
    qc0, kc0, _, _ = run_select(w, p, q, k, ps)
    rng = np.random.default_rng(1)
    h = 1e-6
    checked = 0
    for name, arr, grad in (("q", q, g["dQ"][0]), ("k", k, g["dK"][0]), ("v", v, g["dV"][0])):
        for _ in range(10):
            i, j = int(rng.integers(64)), int(rng.integers(8))
            vals = []
            for sgn in (1, -1):
                a = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                a[name][i, j] += sgn * h
                qc, kc, _, _ = run_select(w, p, a["q"], a["k"], ps)
                if not (np.array_equal(qc, qc0) and np.array_equal(kc, kc0)):
                    vals = None
                    break
                vals.append(_loss(p, a["q"], a["k"], a["v"], do, ps, pl, lam, gs, gl))
            if vals is None:
                continue
            fd = (vals[0] - vals[1]) / (2 * h)
            assert abs(fd - grad[i, j]) <= 1e-6 * max(1.0, abs(fd)), (name, i, j, fd, grad[i, j])
            checked += 1
    assert checked >= 25
    fd = (_loss(p, q, k, v, do, ps, pl, lam + h, gs, gl) - _loss(p, q, k, v, do, ps, pl, lam - h, gs, gl)) / (2 * h)
    assert abs(fd - g["dlambda"][0]) <= 1e-6 * max(1.0, abs(fd))
    for name, arr, grad in (("gs", gs, g["dg_s"][0]), ("gl", gl, g["dg_lr"][0])):
        for i in rng.integers(0, 64, 5):
            a1, a2 = arr.copy(), arr.copy()
            a1[i] += h
            a2[i] -= h
            lp = _loss(p, q, k, v, do, ps, pl, lam, *(a1 if name == "gs" else gs, gl if name == "gs" else a1))
            lm = _loss(p, q, k, v, do, ps, pl, lam, *(a2 if name == "gs" else gs, gl if name == "gs" else a2))
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(fd))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_dense_autograd(causal):
    w = small(causal, N=128, d=16, block=16, r=32)
    p = ref.RefParams.from_workload(w)
    q, k, v, do, ps, pl = head(w, 61)
    gs, gl = (x[0, 0].double() for x in W.gen_gates(w, 61))
    _, _, qp, kp = run_select(w, p, q, k, ps)
    M = D.support_mask(128, 16, causal, qp[0], kp[0])
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    lam = torch.tensor(1.3, dtype=torch.float64, requires_grad=True)
    tgs, tgl = gs.clone().requires_grad_(True), gl.clone().requires_grad_(True)
    dn = D.dense_forward(tq, tk, tv, M, torch.from_numpy(pl[0]), lam, causal, 0.25, g_s=tgs, g_lr=tgl)
    (dn["O"] * torch.from_numpy(do)).sum().backward()
    g = ref.backward(p, q[None], k[None], v[None], do[None], ps, pl, np.array([1.3]),
                     gs.numpy()[None], gl.numpy()[None])
    for a, b in ((g["dQ"][0], tq.grad), (g["dK"][0], tk.grad), (g["dV"][0], tv.grad),
                 (g["dg_s"][0], tgs.grad), (g["dg_lr"][0], tgl.grad)):
        np.testing.assert_allclose(a, b.numpy(), atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(g["dlambda"][0], lam.grad.item(), rtol=1e-9)


def test_backward_with_large_scores_matches_dense_autograd():
    """Scores in the hundreds (lse up to about 450), where d_sparse = exp(lse)
    squared exceeds the fp64 range, with lambda large enough that Eq. 5's ratio m
    takes every value in (0, 1) across the rows: the oracle stays finite and agrees
    with autograd of the dense formulation (Eq. 5 as a logistic function there)."""
    w = small(True, N=128, d=16, block=16, r=32)
    sc = 45.0
    p = ref.RefParams.from_workload(w, scale=sc)
    q, k, v, do, ps, pl = head(w, 67)
    lam_v = 1e150
    _, _, qp, kp = run_select(w, p, q, k, ps)
    M = D.support_mask(128, 16, True, qp[0], kp[0])
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    lam = torch.tensor(lam_v, dtype=torch.float64, requires_grad=True)
    dn = D.dense_forward(tq, tk, tv, M, torch.from_numpy(pl[0]), lam, True, sc, logistic=True)
    m = dn["m"].detach().numpy()
    assert dn["lse"].max().item() > 354.0 and m.min() < 0.05 and m.max() > 0.95
    (dn["O"] * torch.from_numpy(do)).sum().backward()
    o = ref.forward(p, q[None], k[None], v[None], ps, pl, np.array([lam_v]))
    g = ref.backward(p, q[None], k[None], v[None], do[None], ps, pl, np.array([lam_v]))
    for x in (o["O"], g["dQ"], g["dK"], g["dV"], g["dg_s"], g["dlambda"]):
        assert np.isfinite(x).all()
    np.testing.assert_allclose(o["O"][0], dn["O"].detach().numpy(), atol=1e-10, rtol=1e-9)
    for a, b in ((g["dQ"][0], tq.grad), (g["dK"][0], tk.grad), (g["dV"][0], tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), atol=1e-8 * np.abs(b.numpy()).max(), rtol=1e-7)
    np.testing.assert_allclose(g["dlambda"][0], lam.grad.item(), rtol=1e-7)


# ----------------------------------------------------------------------------- learnable gates

def _gate_params(d, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(0, 0.3, (1, 2, d)), rng.normal(0, 0.5, (1, 2))


def test_gates_closed_forms():
    """W = 0, b = 0 gives 1/2; the logistic symmetry g(Q, W, b) + g(-Q, W, -b) = 1;
    a zero query row gives sigmoid(b)."""
    w = small(True, N=64, d=16, block=16)
    p = ref.RefParams.from_workload(w)
    q, *_ = head(w, 71)
    W, b = _gate_params(16, 71)
    gs, gl = ref.gates_fwd(p, q[None], np.zeros_like(W), np.zeros_like(b))
    assert np.all(gs == 0.5) and np.all(gl == 0.5)
    g1 = ref.gates_fwd(p, q[None], W, b)
    g2 = ref.gates_fwd(p, -q[None], W, -b)
    for a, c in zip(g1, g2):
        np.testing.assert_allclose(a + c, 1.0, rtol=0, atol=1e-15)
    q0 = q.copy()
    q0[5] = 0.0
    gs, gl = ref.gates_fwd(p, q0[None], W, b)
    assert gs[0, 5] == 1 / (1 + math.exp(-b[0, 0])) and gl[0, 5] == 1 / (1 + math.exp(-b[0, 1]))


@pytest.mark.parametrize("causal", [False, True])
def test_gated_operator_matches_dense_autograd(causal):
    """Gates from the query's projection composed with the operator: ref_bwd's
    dg_s, dg_lr taken through ref_gates_bwd give the same dQ, dW, db as autograd
    of the dense fp64 formulation with the gates computed there."""
    w = small(causal, N=128, d=16, block=16, r=32)
    p = ref.RefParams.from_workload(w)
    q, k, v, do, ps, pl = head(w, 73)
    W, b = _gate_params(16, 73)
    _, _, qp, kp = run_select(w, p, q, k, ps)
    M = D.support_mask(128, 16, causal, qp[0], kp[0])
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    tW = torch.from_numpy(W[0]).clone().requires_grad_(True)
    tb = torch.from_numpy(b[0]).clone().requires_grad_(True)
    tg = torch.sigmoid(tq @ tW.t() + tb)
    dn = D.dense_forward(tq, tk, tv, M, torch.from_numpy(pl[0]), 1.1, causal, 0.25,
                         g_s=tg[:, 0], g_lr=tg[:, 1])
    (dn["O"] * torch.from_numpy(do)).sum().backward()
    gs, gl = ref.gates_fwd(p, q[None], W, b)
    g = ref.backward(p, q[None], k[None], v[None], do[None], ps, pl, np.array([1.1]), gs, gl)
    dq_gate, dW, db = ref.gates_bwd(p, q[None], W, b, g["dg_s"], g["dg_lr"])
    np.testing.assert_allclose(g["dQ"][0] + dq_gate[0], tq.grad.numpy(), atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(g["dK"][0], tk.grad.numpy(), atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(dW[0], tW.grad.numpy(), atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(db[0], tb.grad.numpy(), atol=1e-10, rtol=1e-9)


def test_gate_gradients_match_central_differences():
    """dW and db of the gate path against central differences of the composed loss
    (the selection does not depend on W, b)."""
    w = small(True, N=64, d=8, block=8, r=32, chunk=16)
    p = ref.RefParams.from_workload(w)
    q, k, v, do, ps, pl = head(w, 79)
    W, b = _gate_params(8, 79)

    def loss(W_, b_):
        gs, gl = ref.gates_fwd(p, q[None], W_, b_)
        return _loss(p, q, k, v, do, ps, pl, 0.8, gs[0], gl[0])

    gs, gl = ref.gates_fwd(p, q[None], W, b)
    g = ref.backward(p, q[None], k[None], v[None], do[None], ps, pl, np.array([0.8]), gs, gl)
    _, dW, db = ref.gates_bwd(p, q[None], W, b, g["dg_s"], g["dg_lr"])
    h = 1e-6
    for kk in range(2):
        for c in range(8):
            a1, a2 = W.copy(), W.copy()
            a1[0, kk, c] += h
            a2[0, kk, c] -= h
            fd = (loss(a1, b) - loss(a2, b)) / (2 * h)
            assert abs(fd - dW[0, kk, c]) <= 1e-6 * max(1.0, abs(fd))
        b1, b2 = b.copy(), b.copy()
        b1[0, kk] += h
        b2[0, kk] -= h
        fd = (loss(W, b1) - loss(W, b2)) / (2 * h)
        assert abs(fd - db[0, kk]) <= 1e-6 * max(1.0, abs(fd))


# ----------------------------------------------------------------------------- exact top-k selector

def _int_qk(N, d, seed, lo=-3, hi=4):
    rng = np.random.default_rng(seed)
    return (rng.integers(lo, hi, (1, N, d)).astype(np.float64),
            rng.integers(lo, hi, (1, N, d)).astype(np.float64))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("k_top", [1, 5, 16, 70])
def test_topk_equals_brute_force_on_exact_integer_scores(causal, k_top):
    """Small-integer rows make every fp64 score exact (and ties frequent): the
    oracle equals a brute force over exact integer dot products ordered by
    (score descending, key index ascending), as ascending sets padded with -1."""
    N, d = 64, 8
    q, k = _int_qk(N, d, 83 + k_top)
    p = ref.RefParams(N=N, d=d, causal=causal, block=N, hash_bits=1, lr_tables=1)
    got = ref.topk(p, q, k, k_top)[0]
    qi, ki = q[0].astype(np.int64), k[0].astype(np.int64)
    for i in range(N):
        cand = range(i + 1) if causal else range(N)
        order = sorted(cand, key=lambda j: (-int(qi[i] @ ki[j]), j))
        want = sorted(order[:k_top])
        want += [-1] * (k_top - len(want))
        assert got[i].tolist() == want, i


def test_topk_ties_take_the_lower_index_and_sets_are_causal():
    """Duplicated keys score equally: the lower indices are taken; causal sets hold
    only keys j <= i, min(k, i + 1) of them."""
    N, d, k_top = 96, 16, 8
    q, k = _int_qk(N, d, 89)
    k[0, 40:80] = k[0, 10]  # 41 copies of key 10's row
    q[0, :] = k[0, 10]      # every query prefers that row
    p = ref.RefParams(N=N, d=d, causal=True, block=N, hash_bits=1, lr_tables=1)
    got = ref.topk(p, q, k, k_top)[0]
    for i in range(N):
        sel = [j for j in got[i] if j >= 0]
        assert len(sel) == min(k_top, i + 1) and all(j <= i for j in sel)
        if i >= 47:  # 10, 40..46 are the 8 lowest copies
            assert sel == [10] + list(range(40, 47)), (i, sel)
    p.causal = False
    assert ref.topk(p, q, k, N + 5)[0, 3].tolist() == list(range(N)) + [-1] * 5


# ----------------------------------------------------------------------------- several hash rounds

def _round_planes(ps, R, seed):
    """R rounds of sortLSH hyperplanes [1, R, bits, d]: round 0 the given ones."""
    rng = np.random.default_rng(seed)
    out = [ps[0]] + [rng.normal(size=ps[0].shape).astype(np.float32) for _ in range(R - 1)]
    return np.stack(out)[None]


@pytest.mark.parametrize("causal", [False, True])
def test_repeated_round_equals_one_round(causal):
    """Two rounds with the same hyperplanes select every pair twice; the union
    counts it once, so the operator equals the one-round operator (forward and
    backward)."""
    w = small(causal, N=128, d=16, block=16, r=32)
    p1 = ref.RefParams.from_workload(w)
    p2 = ref.RefParams.from_workload(w, hash_rounds=2)
    q, k, v, do, ps, pl = head(w, 97)
    ps2 = np.stack([ps[0], ps[0]])[None]
    o1 = ref.forward(p1, q[None], k[None], v[None], ps, pl, np.array([0.7]))
    o2 = ref.forward(p2, q[None], k[None], v[None], ps2, pl, np.array([0.7]))
    for n in ("O", "O_s", "lse"):
        np.testing.assert_allclose(o2[n], o1[n], rtol=1e-12, atol=1e-12)
    g1 = ref.backward(p1, q[None], k[None], v[None], do[None], ps, pl, np.array([0.7]))
    g2 = ref.backward(p2, q[None], k[None], v[None], do[None], ps2, pl, np.array([0.7]))
    for n in ("dQ", "dK", "dV", "dlambda"):
        np.testing.assert_allclose(g2[n], g1[n], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("R", [2, 3])
def test_rounds_union_matches_dense_masked_softmax_and_autograd(causal, R):
    """Several rounds: the sparse branch is the softmax over the union of the
    rounds' supports (dense brute force with the OR of each round's mask), and the
    backward equals autograd of the dense formulation over that mask."""
    w = small(causal, N=128, d=16, block=16, r=32)
    p = ref.RefParams.from_workload(w, hash_rounds=R)
    q, k, v, do, ps, pl = head(w, 101 + R)
    psR = _round_planes(ps, R, 7 + R)
    _, _, qp, kp = ref.select(p, q[None], k[None], psR)
    masks = [D.support_mask(128, 16, causal, qp[0, r], kp[0, r]) for r in range(R)]
    M = np.logical_or.reduce(masks)
    assert M.sum() > max(m.sum() for m in masks) and M.sum() <= sum(m.sum() for m in masks)
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    dn = D.dense_forward(tq, tk, tv, M, torch.from_numpy(pl[0]), 1.2, causal, 0.25)
    o = ref.forward(p, q[None], k[None], v[None], psR, pl, np.array([1.2]))
    for n in ("O", "O_s", "lse", "d_lr"):
        np.testing.assert_allclose(o[n][0], dn[n].detach().numpy(), atol=1e-10, rtol=1e-9)
    (dn["O"] * torch.from_numpy(do)).sum().backward()
    g = ref.backward(p, q[None], k[None], v[None], do[None], psR, pl, np.array([1.2]))
    for a, b in ((g["dQ"][0], tq.grad), (g["dK"][0], tk.grad), (g["dV"][0], tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), atol=1e-10, rtol=1e-9)


# ----------------------------------------------------------------------------- extra edges (Omega_safe)

def _extra_list(N, E, causal, seed, qp=None, kp=None, s=None):
    """[N, E] int32 extra keys per query with every kind of entry the definition
    covers: random keys, -1 padding, out-of-range keys, a key listed twice, keys
    after the query (ignored when causal) and a key sortLSH already selected."""
    rng = np.random.default_rng(seed)
    ex = rng.integers(0, N, size=(N, E)).astype(np.int32)
    ex[:, 1] = -1
    ex[::3, 2] = N + 5
    ex[:, 3] = ex[:, 0]
    ex[:, 4] = np.minimum(np.arange(N) + 3, N - 1)
    ex[:, 5] = np.arange(N)  # the query itself: in its causal leaf
    return ex


def _extra_mask(N, causal, ex):
    M = np.zeros((N, N), bool)
    for i in range(N):
        for j in ex[i]:
            if 0 <= j < N and (not causal or j <= i):
                M[i, j] = True
    return M


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("R", [1, 2])
def test_extra_edges_union_matches_dense_masked_softmax_and_autograd(causal, R):
    """Extra edges (Appendix C's Omega = Omega_LSH u Omega_safe): the sparse branch
    is the softmax over the union of the sortLSH support and the valid listed keys
    (a set: duplicates and keys sortLSH already holds count once; -1, out-of-range
    and, causal, later keys are ignored), checked against dense brute force over
    that mask built here from the definition, and the backward against autograd."""
    N, s, E = 128, 16, 7
    w = small(causal, N=N, d=16, block=s, r=32)
    p = ref.RefParams.from_workload(w, hash_rounds=R, extra_edges=E)
    q, k, v, do, ps, pl = head(w, 211 + R + 2 * causal)
    psR = _round_planes(ps, R, 17 + R) if R > 1 else ps
    _, _, qp, kp = ref.select(p, q[None], k[None], psR)
    lsh = [D.support_mask(N, s, causal, (qp[0, r] if R > 1 else qp[0]),
                          (kp[0, r] if R > 1 else kp[0])) for r in range(R)]
    ex = _extra_list(N, E, causal, 5 + R)
    M0 = np.logical_or.reduce(lsh)
    M = M0 | _extra_mask(N, causal, ex)
    assert M.sum() > M0.sum()
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    dn = D.dense_forward(tq, tk, tv, M, torch.from_numpy(pl[0]), 0.8, causal, 0.25)
    o = ref.forward(p, q[None], k[None], v[None], psR, pl, np.array([0.8]), extra=ex[None])
    for n in ("O", "O_s", "lse", "d_lr"):
        np.testing.assert_allclose(o[n][0], dn[n].detach().numpy(), atol=1e-10, rtol=1e-9)
    (dn["O"] * torch.from_numpy(do)).sum().backward()
    g = ref.backward(p, q[None], k[None], v[None], do[None], psR, pl, np.array([0.8]),
                     extra=ex[None])
    for a, b in ((g["dQ"][0], tq.grad), (g["dK"][0], tk.grad), (g["dV"][0], tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), atol=1e-10, rtol=1e-9)


@pytest.mark.parametrize("causal", [False, True])
def test_extra_edges_listing_every_key_is_exact_attention(causal):
    """Listing every key for every query makes the support all keys (at or before
    the query when causal), so the sparse branch is exact softmax attention,
    whatever sortLSH selected."""
    N, E = 64, 64
    w = small(causal, N=N, d=16, block=16, r=32)
    p = ref.RefParams.from_workload(w, extra_edges=E)
    q, k, v, do, ps, pl = head(w, 223 + causal)
    ex = np.tile(np.arange(N, dtype=np.int32), (N, 1))
    o = ref.forward(p, q[None], k[None], v[None], ps, pl, np.array([1.0]), extra=ex[None])
    S = (q @ k.T) * p.scale if p.scale else (q @ k.T) / math.sqrt(16)
    if causal:
        S = np.where(np.tril(np.ones((N, N), bool)), S, -np.inf)
    lse = np.log(np.exp(S - S.max(1, keepdims=True)).sum(1)) + S.max(1)
    Pm = np.exp(S - lse[:, None])
    np.testing.assert_allclose(o["lse"][0], lse, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o["O_s"][0], Pm @ v, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_extra_edges_already_selected_change_nothing(causal):
    """Extra edges that sortLSH already selects (each query's own causal-leaf keys,
    or the keys of its own block) leave the operator unchanged: the support is a
    set."""
    N, s, E = 128, 16, 4
    w = small(causal, N=N, d=16, block=s, r=32)
    p0 = ref.RefParams.from_workload(w)
    p1 = ref.RefParams.from_workload(w, extra_edges=E)
    q, k, v, do, ps, pl = head(w, 229 + causal)
    _, _, qp, kp = ref.select(p0, q[None], k[None], ps)
    M = D.support_mask(N, s, causal, qp[0], kp[0])
    ex = np.full((N, E), -1, np.int32)
    for i in range(N):
        js = np.flatnonzero(M[i])[:E]
        ex[i, :len(js)] = js
    o0 = ref.forward(p0, q[None], k[None], v[None], ps, pl, np.array([0.6]))
    o1 = ref.forward(p1, q[None], k[None], v[None], ps, pl, np.array([0.6]), extra=ex[None])
    for n in ("O", "O_s", "lse"):
        np.testing.assert_allclose(o1[n], o0[n], rtol=1e-12, atol=1e-13)
    g0 = ref.backward(p0, q[None], k[None], v[None], do[None], ps, pl, np.array([0.6]))
    g1 = ref.backward(p1, q[None], k[None], v[None], do[None], ps, pl, np.array([0.6]),
                      extra=ex[None])
    for n in ("dQ", "dK", "dV", "dlambda"):
        np.testing.assert_allclose(g1[n], g0[n], rtol=1e-10, atol=1e-12)
