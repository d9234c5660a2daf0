"""GPU test of elsaa_select_noalloc, the selection for callers that cannot
allocate (its scratch is a fixed device array): called through the C ABI twice
in a row, the second time with a smaller problem, its codes and orders equal
elsaa_select's (with a caller workspace) bit for bit."""
from __future__ import annotations

import pytest
import torch

import workloads as W
from parity_util import cfg_of, to_dev, wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

CALLS = [
    # causal bf16, 6-bit codes: 8 * 4 * 6 * 128 = 24 KiB of scratch
    wl("a", 2, 4, 4096, 128, "bf16", True, 64, 32, "clusters", n_clusters=32, sigma=0.5),
    # then a smaller non-causal fp32 problem (5-bit codes, d 64)
    wl("b", 1, 2, 1024, 64, "f32", False, 32, 16),
]


def test_noalloc_select_matches_select_twice_in_a_row():
    import sparse_rank_approximation_amd as S
    results = []
    for i, w in enumerate(CALLS):
        print(f"[gpu noalloc] call {i}: {w}", flush=True)
        inp = W.gen_inputs(w, 900 + i, with_do=False)
        d = to_dev({k: inp[k] for k in ("q", "k", "planes_s")})
        cfg = cfg_of(w)
        got = S.select_noalloc(cfg, d["q"], d["k"], d["planes_s"])
        ref = S.select(cfg, d["q"], d["k"], d["planes_s"])
        torch.cuda.synchronize()
        results.append((got, ref))
    for i, (got, ref) in enumerate(results):
        for name, a, b in zip(("q_code", "k_code", "q_perm", "k_perm"), got, ref):
            assert torch.equal(a, b), f"call {i}: {name} differs"
