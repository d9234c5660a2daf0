"""Seeded synthetic inputs for the ELSAA attention operator.

This module is shared by the tests, the benchmark and the oracle checks. It
holds no arithmetic of the operator itself: it only draws Q, K, V, dO, the
hyperplanes, gates and lambda, with the shapes and structure of the paper's
long-context training workloads (text at 16K-64K tokens, tokenised vision),
which stand in for its datasets (ArXiv, Tiny ImageNet, ...) that are not
available here.

Every head (b, h) is drawn from its own generator, seeded from
(seed, b, h, tensor id), so that any subset of heads can be regenerated exactly
without drawing the others.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

BASE_SEED = 20260722


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    block: int          # sortLSH block size s ("k selected keys per query")
    r: int              # RACE feature count L * 2^lr_bits
    gen: str            # Q/K generator kind
    gen_args: dict = field(default_factory=dict)
    lr_bits: int = 4
    chunk: int = 2048   # causal RACE summary spacing (rounding only); sets the walks' parallelism

    @property
    def hash_bits(self) -> int:
        return max(1, int(round(math.log2(self.N // self.block))))

    @property
    def lr_tables(self) -> int:
        return self.r >> self.lr_bits

    @property
    def levels(self) -> int:
        return int(round(math.log2(self.N // self.block))) if self.causal else 1

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload("tiny_single_head_B1_H1_N256_d32_f32", 1, 1, 256, 32, "f32", False, 16, 16,
                "iid", chunk=64),
    2: Workload("gpt2_small_layer_B8_H12_N4096_d64_bf16_causal", 8, 12, 4096, 64, "bf16", True,
                64, 64, "clusters", dict(n_clusters=64, sigma=0.3), chunk=512),
    3: Workload("llama_long_context_B2_H32_N16384_d128_bf16_causal", 2, 32, 16384, 128, "bf16",
                True, 128, 128, "clusters_diffuse",
                dict(n_clusters=256, sigma=0.5, diffuse=0.2), chunk=4096),
    4: Workload("very_long_context_B1_H8_N65536_d128_bf16_causal", 1, 8, 65536, 128, "bf16", True,
                256, 256, "ar1_clusters", dict(n_clusters=1024, rho=0.9, jitter=0.1)),
    5: Workload("vit_batch_B64_H12_N1024_d64_bf16", 64, 12, 1024, 64, "bf16", False, 32, 32,
                "smooth_field", dict(grid=32, blur=2.0, noise=0.3)),
}


def workload_seed(idx: int) -> int:
    return BASE_SEED + idx


def _gen(seed: int, *key: int) -> torch.Generator:
    ss = np.random.SeedSequence([seed & 0xFFFFFFFF, *[int(k) & 0xFFFFFFFF for k in key]])
    g = torch.Generator()
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF))
    return g


def _randn(g: torch.Generator, *shape: int) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def _blur_field(g: torch.Generator, grid: int, sigma: float, channels: int) -> torch.Tensor:
    """`channels` independent grid x grid N(0,1) fields, Gaussian-blurred with
    reflect padding, renormalised to unit variance; returns [grid*grid, channels]
    in raster order."""
    f = _randn(g, channels, grid, grid).double()
    rad = int(math.ceil(4 * sigma))
    x = torch.arange(-rad, rad + 1, dtype=torch.float64)
    w = torch.exp(-0.5 * (x / sigma) ** 2)
    w = w / w.sum()
    f = torch.nn.functional.pad(f[None], (rad, rad, rad, rad), mode="reflect")[0]
    f = torch.nn.functional.conv2d(f[:, None], w.view(1, 1, 1, -1))
    f = torch.nn.functional.conv2d(f, w.view(1, 1, -1, 1))[:, 0]
    f = (f - f.mean(dim=(1, 2), keepdim=True)) / f.std(dim=(1, 2), keepdim=True)
    return f.reshape(channels, grid * grid).t().float()


def gen_qk(w: Workload, seed: int, b: int, h: int) -> tuple[torch.Tensor, torch.Tensor]:
    """Q, K of head (b, h) as fp32 [N, d]. A token's query and key share its
    centroid (or field value) and carry independent noise."""
    g = _gen(seed, b, h, 0)
    N, d, a = w.N, w.d, w.gen_args
    if w.gen == "iid":
        return _randn(g, N, d), _randn(g, N, d)
    if w.gen == "clusters":
        mu = _randn(g, a["n_clusters"], d)
        cid = torch.randint(0, a["n_clusters"], (N,), generator=g)
        s = a["sigma"]
        return mu[cid] + s * _randn(g, N, d), mu[cid] + s * _randn(g, N, d)
    if w.gen == "clusters_diffuse":
        mu = _randn(g, a["n_clusters"], d)
        cid = torch.randint(0, a["n_clusters"], (N,), generator=g)
        diffuse = torch.rand(N, generator=g) < a["diffuse"]
        s = a["sigma"]
        q = mu[cid] + s * _randn(g, N, d)
        k = mu[cid] + s * _randn(g, N, d)
        q[diffuse] = _randn(g, int(diffuse.sum()), d)
        k[diffuse] = _randn(g, int(diffuse.sum()), d)
        return q, k
    if w.gen == "ar1_clusters":
        mu = _randn(g, a["n_clusters"], d)
        cid = torch.randint(0, a["n_clusters"], (N,), generator=g)
        rho = a["rho"]
        xi = _randn(g, N, d).double()
        u = torch.empty(N, d, dtype=torch.float64)
        u[0] = xi[0]
        c = math.sqrt(1.0 - rho * rho)
        # AR(1) along the sequence: u_t = rho u_{t-1} + sqrt(1 - rho^2) xi_t.
        for t in range(1, N):
            u[t] = rho * u[t - 1] + c * xi[t]
        u = u.float()
        j = a["jitter"]
        return mu[cid] + u + j * _randn(g, N, d), mu[cid] + u + j * _randn(g, N, d)
    if w.gen == "smooth_field":
        grid = a["grid"]
        assert grid * grid == N
        f = _blur_field(g, grid, a["blur"], d)
        s = a["noise"]
        return f + s * _randn(g, N, d), f + s * _randn(g, N, d)
    raise ValueError(w.gen)


def gen_v(w: Workload, seed: int, b: int, h: int) -> torch.Tensor:
    return _randn(_gen(seed, b, h, 1), w.N, w.d)


def gen_do(w: Workload, seed: int, b: int, h: int) -> torch.Tensor:
    return _randn(_gen(seed, b, h, 2), w.N, w.d)


def gen_planes(w: Workload, seed: int) -> tuple[torch.Tensor, torch.Tensor]:
    """sortLSH hyperplanes [H, hash_bits, d] and RACE hyperplanes
    [H, lr_tables, lr_bits, d], iid N(0,1) fp32, one set per head shared by the
    batch."""
    ps = torch.stack([_randn(_gen(seed + 1, h), w.hash_bits, w.d) for h in range(w.H)])
    plr = torch.stack([_randn(_gen(seed + 2, h), w.lr_tables, w.lr_bits, w.d) for h in range(w.H)])
    return ps.contiguous(), plr.contiguous()


def gen_planes_rounds(w: Workload, seed: int, rounds: int) -> torch.Tensor:
    """sortLSH hyperplanes for several hash rounds, [H, rounds, hash_bits, d]:
    round 0 is gen_planes' set, round u > 0 is drawn from its own generator."""
    per = []
    for h in range(w.H):
        per.append(torch.stack([_randn(_gen(seed + 1 + 100 * u, h), w.hash_bits, w.d)
                                for u in range(rounds)]))
    return torch.stack(per).contiguous()


def gen_extra_edges(w: Workload, seed: int, E: int, pad: float = 0.25) -> torch.Tensor:
    """Extra keys per query, int32 [B, H, N, E]: a stand-in for the Bernoulli draw
    of Appendix C's Omega_safe. Each entry is a key drawn uniformly from the keys
    the query may see (all N, or 0..i when causal), replaced by -1 padding with
    probability `pad`; entry 1 repeats entry 0 (a key listed twice)."""
    g = _gen(seed + 5, 0)
    B, H, N = w.B, w.H, w.N
    u = torch.rand(B, H, N, E, generator=g, dtype=torch.float64)
    hi = (torch.arange(N, dtype=torch.float64) + 1.0)[None, None, :, None] if w.causal else float(N)
    ex = torch.minimum(torch.floor(u * hi), torch.as_tensor(N - 1.0)).to(torch.int32)
    drop = torch.rand(B, H, N, E, generator=g) < pad
    ex = torch.where(drop, torch.full_like(ex, -1), ex)
    if E > 1:
        ex[..., 1] = ex[..., 0]
    return ex.contiguous()


def gen_gates(w: Workload, seed: int) -> tuple[torch.Tensor, torch.Tensor]:
    g = _gen(seed + 3, 0)
    gs = 0.5 + torch.rand(w.B, w.H, w.N, generator=g)
    glr = 0.5 + torch.rand(w.B, w.H, w.N, generator=g)
    return gs, glr


def gen_lambda(w: Workload, seed: int, random: bool = False) -> torch.Tensor:
    if not random:
        return torch.ones(w.H)
    return 0.25 + 2.0 * torch.rand(w.H, generator=_gen(seed + 4, 0))


def gen_inputs(w: Workload, seed: int, heads=None, with_do: bool = True) -> dict:
    """Q, K, V (and dO) [B, H, N, d] in the workload dtype, on the CPU.
    `heads`: optional list of (b, h) to draw; other heads are left zero."""
    dt = w.torch_dtype
    out = {k: torch.zeros(w.B, w.H, w.N, w.d, dtype=dt) for k in ("q", "k", "v")}
    if with_do:
        out["do"] = torch.zeros(w.B, w.H, w.N, w.d, dtype=dt)
    todo = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in todo:
        q, k = gen_qk(w, seed, b, h)
        out["q"][b, h] = q.to(dt)
        out["k"][b, h] = k.to(dt)
        out["v"][b, h] = gen_v(w, seed, b, h).to(dt)
        if with_do:
            out["do"][b, h] = gen_do(w, seed, b, h).to(dt)
    out["planes_s"], out["planes_lr"] = gen_planes(w, seed)
    return out
