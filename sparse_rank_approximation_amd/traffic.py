"""Memory traffic per kernel from rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE).

Two roles, one per step of the measurement:

    python -m sparse_rank_approximation_amd.traffic copy
        A plain device copy of COPY_BYTES (torch's copy kernel), the calibration
        workload: run it under `rocprofv3 --pmc FETCH_SIZE` and again under
        `--pmc WRITE_SIZE`. It reads and writes exactly COPY_BYTES, so the ratio
        COPY_BYTES / counter converts the counters to bytes.

    python -m sparse_rank_approximation_amd.traffic summarize OUT.json \\
        FETCH_BENCH.csv WRITE_BENCH.csv FETCH_COPY.csv WRITE_COPY.csv [WORKLOAD]
        Reads the counter_collection CSVs of the four runs (the bench.py runs and
        the copy runs) and writes OUT.json: per kernel, the average FETCH_SIZE and
        WRITE_SIZE per dispatch, the calibration factors and the calibrated bytes
        per launch, tagged with the workload they were taken on (default: the
        B2 H32 N16384 d128 bf16 causal one that bench.py runs by default) and the
        hash of the built library they were taken with (bench.py uses the figures
        only for that workload and while that library is the one it loads: a
        change to a kernel or to a launch changes it, a comment does not).
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import sys

COPY_BYTES = 1 << 30  # 1 GiB read + 1 GiB written: well past the last-level cache

PKG = os.path.dirname(os.path.abspath(__file__))


def library_hash():
    """First 16 hex digits of the SHA-256 of the built library; None if not built."""
    from sparse_rank_approximation_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        return None
    return hashlib.sha256(open(_lib.LIB_PATH, "rb").read()).hexdigest()[:16]


def short_name(name: str):
    """The library's launch name of a kernel symbol; None for kernels of other libraries."""
    if "elsaa" not in name:
        return None
    if "combine_kernel" in name:
        return "combine_q" if "ELb1" in name else "combine_kv"
    if "topk_stream_kernel" in name:  # (the radix passes, then the listing pass)
        return "topk_collect" if "ELb1" in name else "topk_thresh"
    # sparse_bwd_kernel<T, D, SB, ROLE, MR>: role 2 is the separate dQ launch
    m = re.search(r"sparse_bwd_kernelI(?:DF16b|f)Li\d+ELi\d+ELi(\d)E", name)
    if m or "sparse_bwd_kernel<" in name:
        role = m.group(1) if m else name.split("sparse_bwd_kernel<")[1].split(",")[3].strip()
        return "sparse_bwd_q" if role == "2" else "sparse_bwd"
    for k, launch in (("topk_heap_kernel", "topk_redo"), ("order_fill_kernel", "check_fill"),
                      ("order_mark_kernel", "check_mark"), ("order_verify_kernel", "check_verify"),
                      ("finite_count_kernel", "check_finite")):
        if k in name:
            return launch
    for k in ("sparse_bwd", "sparse_fwd", "lr_bwd_k", "lr_bwd_q", "fwd_epilogue", "lr_sums",
              "lr_scan", "hash_kernel", "sort_small_kernel", "sort_kernel", "merge_kernel", "bwd_rows", "dlam_reduce",
              "planes_transpose", "planes_f64", "block_ids", "extra_prep", "extra_fwd",
              "extra_bwd_q", "extra_bwd_k", "radix_hist", "radix_scan", "radix_scatter",
              "topk_finish", "topk_heap", "topk_zero", "gates_fwd", "gates_bwd", "gates_reduce",
              "fused_fwd"):
        if k in name:
            return k.replace("_kernel", "").replace("planes_transpose", "planes_t")
    return name.split("(")[0][-48:]


def per_dispatch(path: str) -> dict:
    """{kernel: (dispatches, mean counter value per dispatch in KiB)}."""
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        if k is None:
            continue
        tot[k] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    return {k: (len(disp[k]), tot[k] / len(disp[k])) for k in tot}


def copy_kib(path: str) -> float:
    """Counter value (KiB) of the largest dispatch of the calibration run."""
    best = 0.0
    vals = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    for v in vals.values():
        best = max(best, v)
    return best


def run_copy() -> None:
    import torch
    n = COPY_BYTES // 2
    src = torch.randn(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes", flush=True)


DEFAULT_WORKLOAD = "llama_long_context_B2_H32_N16384_d128_bf16_causal"


def summarize(out, fb, wb, fc, wc, workload=DEFAULT_WORKLOAD) -> None:
    f_bench, w_bench = per_dispatch(fb), per_dispatch(wb)
    kf = COPY_BYTES / (copy_kib(fc) * 1024.0)
    kw = COPY_BYTES / (copy_kib(wc) * 1024.0)
    kernels = {}
    for k in sorted(set(f_bench) | set(w_bench)):
        fk = f_bench.get(k, (0, 0.0))[1]
        wk = w_bench.get(k, (0, 0.0))[1]
        kernels[k] = {"fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wk, 1),
                      "hbm_bytes_per_launch": round(fk * 1024.0 * kf + wk * 1024.0 * kw)}
    rec = {"library_hash": library_hash(), "workload": workload, "copy_bytes": COPY_BYTES,
           "fetch_factor": round(kf, 4), "write_factor": round(kw, 4), "kernels": kernels}
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "copy":
        run_copy()
    elif len(sys.argv) in (7, 8) and sys.argv[1] == "summarize":
        summarize(*sys.argv[2:])
    else:
        print(__doc__)
        sys.exit(2)
