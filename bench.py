#!/usr/bin/env python3
"""ELSAA attention, forward + backward, on one MI355X.

One step is the whole hot path over one batch of resident synthetic inputs:
elsaa_select (hash + sort), elsaa_lowrank_summary, elsaa_fwd and elsaa_bwd.
Prints one JSON line: whole-job tokens/s (B * N tokens per fwd+bwd step, timed
with no instrumentation), the roofline fraction of the dominant kernel (timed
with HIP events on its launch stream through the library's diagnostics, in a
second pass), the whole step's fraction of its own roofline, and the oracle
timed on this host's cores on a bounded sample of heads.

    python bench.py [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ELSAA fwd+bwd tokens/sec at N=16k,d_h=128 bf16 on 1 GPU; % of roofline"
UNIT = "tokens/s"
# MI355X published peaks.
PEAK_HBM_GBS = 8000.0
PEAK_MFMA = {"bf16": 2500.0, "f32": 157.3}  # dense TFLOP/s
PEAK_FP64_VECTOR = 78.6


def selected_pairs(w, rounds: int = 1) -> int:
    """Query-key pairs of the sparse branch per head (the support sizes summed).
    With several hash rounds, the pairs of every round's blocks (the kernels form
    each round's blocks in full and mask the pairs an earlier round holds)."""
    if not w.causal:
        return rounds * w.N * w.block
    lv = int(round(math.log2(w.N // w.block)))
    return rounds * lv * (w.N // 2) * w.block + w.N * (w.block + 1) // 2


def kernel_work(w, rounds: int = 1) -> dict:
    """Algorithmic work per launch of each kernel: (bound, amount, unit).
    Flops count the contractions the method needs (not masked-tile waste or
    recomputation); bytes count compulsory reads and writes of that kernel."""
    BH, N, d, r = w.B * w.H, w.N, w.d, w.r
    e = 2 if w.dtype == "bf16" else 4
    pairs = selected_pairs(w, rounds) * BH
    tok = BH * N
    return {
        "sparse_fwd": ("mfma", 4.0 * d * pairs, "TFLOP/s"),
        "sparse_bwd": ("mfma", 8.0 * d * pairs, "TFLOP/s"),
        "fwd_epilogue": ("mfma", 2.0 * r * (d + 1) * tok, "TFLOP/s"),
        "lr_sums": ("mfma", 2.0 * r * (d + 1) * tok, "TFLOP/s"),
        "lr_bwd_q": ("mfma", 2.0 * r * (d + 1) * tok, "TFLOP/s"),
        "lr_bwd_k": ("mfma", 4.0 * r * (d + 1) * tok, "TFLOP/s"),
        "hash": ("hbm", 2.0 * tok * d * e + 4.0 * tok, "GB/s"),
        "bwd_rows": ("hbm", 3.0 * tok * d * e + 40.0 * tok, "GB/s"),
        "gates_fwd": ("hbm", tok * d * e + 8.0 * tok, "GB/s"),
        "gates_bwd": ("hbm", 3.0 * tok * d * e + 16.0 * tok, "GB/s"),
        # the one-launch forward: reads Q, K, V; writes O, O_lr (dtype), O_s (fp32),
        # lse, d_lr, two codes and two order entries per token-head
        "fused_fwd": ("hbm", tok * (5.0 * d * e + 4.0 * d + 20.0), "GB/s"),
    }


def step_work(w, rounds: int = 1) -> tuple[float, float]:
    """Algorithmic flops and bytes of one fwd+bwd step over the whole batch.
    Flops: 4 d per selected pair in the forward and 8 d in the backward; per token
    4 r (d + 1) + 4 d L gamma for the low-rank branch in the forward, twice that in
    the backward. Bytes: each token-head reads Q, K, V and writes O, lse, d_lr
    (forward), reads Q, K, V, O, dO and its row statistics and writes dQ, dK, dV
    (backward): 12 d e + 16; plus its two codes (4) and its share of the two
    orders, written once and read twice (3 x 8 P / N)."""
    BH, N, d, r = w.B * w.H, w.N, w.d, w.r
    e = 2 if w.dtype == "bf16" else 4
    tok = BH * N
    perm_len = rounds * (w.levels * (N // 2) if w.causal else N)
    flops = 12.0 * d * selected_pairs(w, rounds) * BH
    flops += 3.0 * tok * (4.0 * r * (d + 1) + 4.0 * d * w.lr_tables * w.lr_bits)
    nbytes = tok * (12.0 * d * e + 16.0 + 4.0 + 3.0 * 8.0 * perm_len / N)
    return flops, nbytes


def roofline(name, launches, total_ms, w, traffic_file, rounds: int = 1, workload=None):
    """workload: the name the committed traffic figures must carry to be used (None:
    a variant run, which they never describe)."""
    work = kernel_work(w, rounds)
    if name not in work:
        return None
    bound, amount, unit = work[name]
    avg_s = total_ms / launches / 1e3
    if bound == "mfma":
        achieved = amount / avg_s / 1e12
        peak = PEAK_MFMA[w.dtype]
    else:
        achieved = amount / avg_s / 1e9
        peak = PEAK_HBM_GBS
    return {"bound": bound, "kernel": name, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "avg_launch_us": round(avg_s * 1e6, 1),
            "traffic": traffic_bytes(name, traffic_file, workload)}


def traffic_bytes(name, path, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on this workload with the library this run loads;
    else None."""
    from sparse_rank_approximation_amd.traffic import library_hash
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    lib = library_hash()
    if lib is None or rec.get("library_hash") != lib or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(name)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(w, seed, n_heads, threads):
    """The oracle (plain fp64 C, OpenMP over heads) on `n_heads` full-size heads:
    select + forward + backward. Scaled to the whole workload's tokens/s."""
    import numpy as np
    import workloads as W
    from oracle import ref
    heads = [((i * 7) % w.B, (i * 5) % w.H) for i in range(n_heads)]
    dt = w.torch_dtype

    def arr(t):
        return t.to(dt).double().numpy()

    q, k, v, do = [], [], [], []
    for b, h in heads:
        qq, kk = W.gen_qk(w, seed, b, h)
        q.append(arr(qq)); k.append(arr(kk))
        v.append(arr(W.gen_v(w, seed, b, h))); do.append(arr(W.gen_do(w, seed, b, h)))
    ps, pl = W.gen_planes(w, seed)
    ps = np.stack([ps[h].numpy() for _, h in heads])
    pl = np.stack([pl[h].numpy() for _, h in heads])
    p = ref.RefParams.from_workload(w)
    ref.lib()
    t0 = time.perf_counter()
    ref.backward(p, np.stack(q), np.stack(k), np.stack(v), np.stack(do), ps, pl, np.ones(n_heads))
    t = time.perf_counter() - t0
    tokens_per_s = n_heads * w.N / (w.H * t)
    return {"value": round(tokens_per_s, 1), "unit": UNIT, "cores": threads,
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{n_heads} of {w.B * w.H} heads at full N={w.N}, select+fwd+bwd in fp64, "
                      f"{t:.1f} s wall on {threads} threads (OpenMP over heads; the host shows "
                      f"{os.cpu_count()} CPUs); scaled by heads"}


def bench_topk(args, w, cfg, d):
    """elsaa_topk at the workload's shape with k = its block size. Its algorithmic
    work is the score of every candidate pair, 2 d flops each on MFMA (the
    contraction the selection needs); the selection forms those scores five times
    (four radix passes and the listing pass) and rescores the listed keys in fp64
    on top."""
    import torch
    import sparse_rank_approximation_amd as S
    from sparse_rank_approximation_amd import _lib
    k_top = w.block
    for _ in range(args.warmup):
        S.topk(cfg, d["q"], d["k"], k_top)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        S.topk(cfg, d["q"], d["k"], k_top)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # Per-kernel times from a second pass with the library's launch events on.
    _lib.profile(True)
    S.topk(cfg, d["q"], d["k"], k_top)
    torch.cuda.synchronize()
    _lib.profile(False)
    rep = _lib.profile_report()
    kernels = {k: {"launches": n, "avg_us": round(t / n * 1e3, 1)} for k, (n, t) in sorted(rep.items())}
    print("[bench] profiled; kernels: " + json.dumps(kernels), file=sys.stderr, flush=True)
    BH, N = w.B * w.H, w.N
    pairs = BH * (N * (N + 1) // 2 if w.causal else N * N)
    flops = 2.0 * w.d * pairs
    achieved = flops / (ms / 1e3) / 1e12
    peak = PEAK_MFMA[w.dtype]
    out = {"metric": "exact per-query top-k selection, queries/s", "value": round(BH * N / (ms / 1e3), 1),
           "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "N": N, "d_h": w.d,
                      "causal": w.causal, "k": k_top},
           "roofline": {"bound": "mfma", "kernel": "topk", "achieved": round(achieved, 2),
                        "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                        "avg_launch_us": round(ms * 1e3, 1), "traffic": None},
           "kernels": kernels}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--topk", action="store_true",
                    help="time elsaa_topk (exact per-query top-k keys, k = the workload's block) "
                         "alone instead of the fwd+bwd step")
    ap.add_argument("--learned-gates", action="store_true",
                    help="gates of Eq. 4 from a learned projection of the query (elsaa_gates_fwd/"
                         "_bwd in every step) instead of unit gates")
    ap.add_argument("--chunk", type=int, default=0,
                    help="causal RACE summary spacing (numerics-neutral); 0 keeps the workload's")
    ap.add_argument("--hash-rounds", type=int, default=1,
                    help="sortLSH hash rounds (the sparse support is the union of theirs)")
    ap.add_argument("--extra-edges", type=int, default=0,
                    help="random extra keys listed per query (Omega_safe) joining the support")
    ap.add_argument("--fused", action="store_true",
                    help="the forward as one launch (elsaa_fwd_fused; non-causal workloads) "
                         "instead of elsaa_select + elsaa_lowrank_summary + elsaa_fwd")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the operator is measured per GPU; heads would shard across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(1)
    threads = min(16, int(os.environ.get("OMP_NUM_THREADS", "16")), os.cpu_count() or 1)
    os.environ["OMP_NUM_THREADS"] = str(threads)

    import torch
    import workloads as W
    import sparse_rank_approximation_amd as S
    from sparse_rank_approximation_amd import _lib

    w = W.WORKLOADS[args.config]
    if args.chunk:
        w = w.with_(chunk=args.chunk)
    seed = W.workload_seed(args.config)
    t0 = time.perf_counter()
    inp = W.gen_inputs(w, seed)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    del inp
    print(f"[bench] inputs for {w.name} ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)
    cfg = S.ElsaaConfig(w.B, w.H, w.N, w.d, w.torch_dtype, w.causal, w.block, w.hash_bits,
                        w.lr_tables, w.lr_bits, w.chunk, hash_rounds=args.hash_rounds,
                        extra_edges=args.extra_edges)
    if args.hash_rounds > 1:
        d["planes_s"] = W.gen_planes_rounds(w, seed, args.hash_rounds).to(dev)
    extra = W.gen_extra_edges(w, seed, args.extra_edges).to(dev) if args.extra_edges else None
    lam = torch.ones(w.H, dtype=torch.float32, device=dev)
    gen = torch.Generator().manual_seed(seed + 5)
    gate_w = (0.2 * torch.randn(w.H, 2, w.d, generator=gen)).to(dev)
    gate_b = (0.5 * torch.randn(w.H, 2, generator=gen)).to(dev)

    def step():
        gs = gl = None
        if args.learned_gates:
            gs, gl = S.gates(cfg, d["q"], gate_w, gate_b)
        if args.fused:
            o = S.forward_fused(cfg, d["q"], d["k"], d["v"], d["planes_s"], d["planes_lr"], lam,
                                gs, gl)
            qp, kp, A, z = o["q_perm"], o["k_perm"], o["A"], o["z"]
        else:
            _, _, qp, kp = S.select(cfg, d["q"], d["k"], d["planes_s"])
            A, z = S.lowrank_summary(cfg, d["k"], d["v"], d["planes_lr"])
            o = S.forward(cfg, d["q"], d["k"], d["v"], d["planes_lr"], qp, kp, A, z, lam, gs, gl,
                          extra=extra)
        g = S.backward(cfg, d["q"], d["k"], d["v"], d["do"], o["O_s"], o["O_lr"], d["planes_lr"],
                       qp, kp, A, z, o["lse"], o["d_lr"], lam, gs, gl, extra=extra)
        if args.learned_gates:
            S.gates_backward(cfg, d["q"], gate_w, gs, gl, g["dg_s"], g["dg_lr"], g["dQ"])

    if args.topk:
        return bench_topk(args, w, cfg, d)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    # The headline: K steps with no instrumentation, between two events on the
    # stream every call enqueues on.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tokens = w.B * w.N
    value = tokens / (ms / 1e3)
    print(f"[bench] timed: {ms:.4f} ms per step", file=sys.stderr, flush=True)
    # Per-kernel times from a second pass with the library's launch events on.
    psteps = max(1, min(args.steps, 10))
    _lib.profile(True)
    for _ in range(psteps):
        step()
    torch.cuda.synchronize()
    _lib.profile(False)
    rep = _lib.profile_report()
    kernels = {k: {"launches": n, "avg_us": round(t / n * 1e3, 1),
                   "ms_per_step": round(t / psteps, 3)} for k, (n, t) in sorted(rep.items())}
    dom = max(rep, key=lambda k: rep[k][1])
    plain = (args.hash_rounds == 1 and args.extra_edges == 0 and not args.learned_gates and
             not args.fused)
    roof = roofline(dom, rep[dom][0], rep[dom][1], w,
                    os.path.join(ROOT, "profiles", "traffic.json"), args.hash_rounds,
                    w.name if plain else None)
    if roof is None:
        roof = {"kernel": dom, "avg_launch_us": round(rep[dom][1] / rep[dom][0] * 1e3, 1)}
    f_alg, b_alg = step_work(w, args.hash_rounds)
    t_roof = max(f_alg / (PEAK_MFMA[w.dtype] * 1e12), b_alg / (PEAK_HBM_GBS * 1e9))
    roof["step_frac"] = round(t_roof / (ms / 1e3), 4)
    roof["step"] = {"flops": f_alg, "bytes": b_alg, "t_roof_us": round(t_roof * 1e6, 1),
                    "bound": "mfma" if f_alg / (PEAK_MFMA[w.dtype] * 1e12) >=
                             b_alg / (PEAK_HBM_GBS * 1e9) else "hbm"}
    print("[bench] profiled; kernels: " + json.dumps(kernels), file=sys.stderr, flush=True)

    cpu = None
    # (the oracle leg times the headline operator; the variants are GPU-only runs)
    if not args.no_cpu_baseline and args.hash_rounds == 1 and args.extra_edges == 0:
        cpu = cpu_baseline(w, seed, min(args.cpu_heads, w.B * w.H), threads)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded generators shaped like the paper's long-context workloads)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d_h": w.d,
                   "causal": w.causal, "block": w.block, "r": w.r, "hash_bits": w.hash_bits,
                   "chunk": w.chunk, "gates": "learned" if args.learned_gates else "unit",
                   "hash_rounds": args.hash_rounds, "extra_edges": args.extra_edges,
                   "forward": "fused" if args.fused else "select+summary+fwd",
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "none"},
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
