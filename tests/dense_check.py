"""Brute-force dense fp64 checks of the ELSAA definitions, used only to pin the
oracle on tiny inputs (N <= 512). Nothing here shares code with the oracle or
with the GPU library.

It builds the explicit N x N support mask from sorted orders (the sparse branch
of "ELSAA: Efficient Low-Rank and Sparse Attention Approximation for Training
Transformers", Section 3.2: diagonal blocks of the permuted score matrix, plus
the causal divide-and-conquer), evaluates softmax attention over it with dense
matrices, evaluates the low-rank branch as the explicit double sum of Section 3.1,
and fuses with Eq. 4 / Eq. 5, all in torch float64 so autograd gives reference
gradients.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np
import torch


def gray(x: int) -> int:
    """Reflected binary Gray code of x."""
    return x ^ (x >> 1)


def gray_rank_table(bits: int) -> np.ndarray:
    """rank[code] = position of `code` along the Gray sequence gray(0), gray(1), ..."""
    t = np.zeros(1 << bits, np.int64)
    for pos in range(1 << bits):
        t[gray(pos)] = pos
    return t


def exact_sign_bits(x: np.ndarray, planes: np.ndarray) -> np.ndarray:
    """Hash code of each row of x from the exact rational sign of <x, plane>."""
    n, bits = x.shape[0], planes.shape[0]
    codes = np.zeros(n, np.int64)
    fp = [[Fraction(float(v)) for v in planes[b]] for b in range(bits)]
    for t in range(n):
        fx = [Fraction(float(v)) for v in x[t]]
        c = 0
        for b in range(bits):
            if sum(a * p for a, p in zip(fx, fp[b])) > 0:
                c |= 1 << b
        codes[t] = c
    return codes


def support_mask(N: int, s: int, causal: bool, qperm: np.ndarray, kperm: np.ndarray) -> np.ndarray:
    """Boolean [N, N]: key j in the support of query i."""
    M = np.zeros((N, N), bool)
    if not causal:
        for b in range(N // s):
            qs = qperm[0, b * s:(b + 1) * s]
            ks = kperm[0, b * s:(b + 1) * s]
            M[np.ix_(qs, ks)] = True
        return M
    for i in range(N):
        lo = (i // s) * s
        M[i, lo:i + 1] = True
    levels = qperm.shape[0]
    for lev in range(levels):
        n = N >> lev
        for a in range(0, N, n):
            off = (a // n) * (n // 2)
            for b in range((n // 2) // s):
                qs = qperm[lev, off + b * s: off + (b + 1) * s]
                ks = kperm[lev, off + b * s: off + (b + 1) * s]
                M[np.ix_(qs, ks)] = True
    return M


def features_torch(x: torch.Tensor, planes: torch.Tensor, scale: float, tau: float) -> torch.Tensor:
    """phi(x) [n, L*2^g]: per table, softmax over the hypercube vertices of
    <v, u>/tau with u = scale * R x (Section 3.1 soft bucket assignment)."""
    L, g, d = planes.shape
    u = scale * torch.einsum("ltd,nd->nlt", planes.double(), x)
    verts = torch.tensor([[1.0 if (b >> t) & 1 else -1.0 for t in range(g)] for b in range(1 << g)],
                         dtype=torch.float64)
    logits = torch.einsum("nlt,bt->nlb", u, verts) / tau
    return torch.softmax(logits, dim=-1).reshape(x.shape[0], L << g)


def dense_forward(q, k, v, mask, planes_lr, lam, causal, scale, tau=1.0, eps=1e-6,
                  g_s=None, g_lr=None, logistic=False):
    """Dense fp64 ELSAA forward of one head. q,k,v torch float64 [N, d].
    logistic: evaluate Eq. 5 as the logistic function of lse - log(lam d_lr + eps)
    (the same value; needed where exp(lse) or its square would overflow)."""
    N = q.shape[0]
    Mt = torch.as_tensor(mask)
    S = (q @ k.t()) * scale
    S = S.masked_fill(~Mt, float("-inf"))
    lse = torch.logsumexp(S, dim=1)
    P = torch.exp(S - lse[:, None])
    O_s = P @ v
    fq = features_torch(q, planes_lr, scale, tau)
    fk = features_torch(k, planes_lr, scale, tau)
    Wl = fq @ fk.t()
    if causal:
        Wl = torch.tril(Wl)
    d_lr = Wl.sum(dim=1)
    O_lr = (Wl @ v) / d_lr[:, None]
    if logistic:
        m = torch.sigmoid(lse - torch.log(lam * d_lr + eps))
    else:
        ds = torch.exp(lse)
        m = ds / (ds + lam * d_lr + eps)
    gs = torch.ones(N, dtype=torch.float64) if g_s is None else g_s
    gl = torch.ones(N, dtype=torch.float64) if g_lr is None else g_lr
    O = (gs * m)[:, None] * O_s + gl[:, None] * O_lr
    return dict(O=O, O_s=O_s, O_lr=O_lr, lse=lse, d_lr=d_lr, m=m)


def popcount(x: int) -> int:
    return bin(x).count("1")
