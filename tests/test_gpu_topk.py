"""GPU parity of elsaa_topk (exact per-query top-k keys on Q K^T, ties to the
lower key index) against the oracle, bit for bit: bf16 and fp32, causal and not,
d_h 32 / 64 / 128, k from 16 to 256, clustered inputs with many near ties, exact
duplicate keys, and k above the causal candidate count (padding). A head whose
keys are all one row ties every score: later queries then list more keys than
their list holds, and their tiles are redone by the heap kernel."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from parity_util import all_heads, cfg_of, head_arrays, to_dev, wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

# name: (workload, k, duplicate key rows)
CASES = {
    "causal_bf16_N4096_d64_k64": (wl("t", 1, 2, 4096, 64, "bf16", True, 64, 16, "clusters",
                                     n_clusters=64, sigma=0.3), 64, False),
    "noncausal_f32_N512_d32_k16": (wl("t", 2, 1, 512, 32, "f32", False, 32, 16), 16, False),
    "causal_bf16_N1024_d128_k128_ties": (wl("t", 1, 2, 1024, 128, "bf16", True, 128, 16, "clusters",
                                            n_clusters=8, sigma=0.5), 128, True),
    "noncausal_bf16_N1024_d128_k256": (wl("t", 1, 1, 1024, 128, "bf16", False, 128, 16), 256, False),
    "causal_f32_N128_d64_k100_padded": (wl("t", 1, 1, 128, 64, "f32", True, 32, 16), 100, True),
    "causal_bf16_N512_d64_k64_all_tied": (wl("t", 1, 2, 512, 64, "bf16", True, 64, 16), 64, "all"),
    # a partial 128-query workgroup and a partial 32-query tile; k = 1
    "noncausal_f32_N96_d32_k8": (wl("t", 1, 1, 96, 32, "f32", False, 32, 16), 8, False),
    "causal_bf16_N64_d128_k1": (wl("t", 1, 2, 64, 128, "bf16", True, 64, 16), 1, False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_topk_parity(case):
    import sparse_rank_approximation_amd as S
    w, k_top, dup = CASES[case]
    print(f"[gpu topk] {case} {w} k={k_top}", flush=True)
    inp = W.gen_inputs(w, 6000 + len(case), with_do=False)
    if dup == "all":  # every key of head 1 the same row: all scores of a query tie
        inp["k"][:, 1] = inp["k"][:, 1, 7:8]
    elif dup:  # a run of exact copies of one key row in every head, and queries close to it
        inp["k"][:, :, w.N // 4: w.N // 4 + w.N // 8] = inp["k"][:, :, 3:4]
        inp["q"][:, :, ::5] = inp["k"][:, :, 3:4]
    d = to_dev({n: inp[n] for n in ("q", "k")})
    idx = S.topk(cfg_of(w), d["q"], d["k"], k_top)
    torch.cuda.synchronize()
    heads = all_heads(w)
    q, k, *_ = head_arrays(w, {**inp, "v": inp["q"], "do": inp["q"]}, heads)
    want = ref.topk(ref.RefParams.from_workload(w), q, k, k_top)
    got = idx.view(len(heads), w.N, k_top).cpu().numpy()
    bad = np.argwhere((got != want).any(axis=2))
    assert bad.size == 0, f"{case}: {len(bad)} queries differ, first {bad[:3].tolist()}"
