"""Host logic of the HBM-traffic calibration (sparse_rank_approximation_amd/traffic.py).

rocprofv3 counter CSVs are written here by hand, in the layout rocprofv3 uses
(one row per dispatch and counter, possibly several rows per dispatch), and the
summary is checked against numbers worked out by hand.
"""
import csv
import json

from sparse_rank_approximation_amd import traffic

HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value in KiB)."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(HEADER)
        for i, (d, name, v) in enumerate(rows):
            w.writerow([i + 1, d, "Agent 1", 1, 1, 1, 256, 7, name, 256, 0, 0, 4, 0, 16, counter,
                        float(v), 0, 1])


# Names as rocprofv3 reports them: template kernels mangled, the others demangled.
COMBINE_Q = "_ZN5elsaa12_GLOBAL__N_114combine_kernelIDF16bLi128ELb1ELi1EEEvPKT_S4_PS2_S5_iii"
COMBINE_KV = "_ZN5elsaa12_GLOBAL__N_114combine_kernelIDF16bLi128ELb0ELi2EEEvPKT_S4_PS2_S5_iii"
HASH = "_ZN5elsaa11hash_kernelIDF16bLi128ELi7EEEvPKT_S3_PKdPtS6_ii"
SPARSE_BWD = "_ZN5elsaa18sparse_bwd2_kernelILi128ELi128EEEvPKDF16bS2_S2_S2_PKfS4_S4_PKiS6_iiifiiPDF16bS7_S7_"


def test_short_names():
    assert traffic.short_name("void at::native::vectorized_elementwise_kernel<4>(int)") is None
    assert traffic.short_name(COMBINE_Q) == "combine_q"
    assert traffic.short_name(COMBINE_KV) == "combine_kv"
    assert traffic.short_name(HASH) == "hash"
    assert traffic.short_name(SPARSE_BWD) == "sparse_bwd"
    assert traffic.short_name("elsaa::planes_f64_kernel(float const*, int, double*)") == "planes_f64"
    assert traffic.short_name("elsaa::planes_transpose_kernel(float const*, int, int, int, float*)") == "planes_t"


def test_every_launch_name_maps_back():
    """Every ELSAA_LAUNCH name in the sources is what short_name gives for its
    kernel, so a counter summary is keyed by the names bench.py reports."""
    import glob
    import os
    import re
    csrc = os.path.join(os.path.dirname(traffic.__file__), "csrc")
    text = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) +
                                                 glob.glob(os.path.join(csrc, "*.cpp"))))
    pairs = set(re.findall(r'ELSAA_LAUNCH\("([a-z_0-9]+)",\s*\(?([A-Za-z_0-9]+)', text))
    assert len(pairs) > 30
    names = {}
    for launch, kern in pairs:
        names.setdefault(kern, set()).add(launch)
    for kern, launches in names.items():
        if len(launches) == 1:  # (kernels launched under several names: below)
            assert traffic.short_name(f"elsaa::{kern}(int)") == next(iter(launches)), kern
    assert {k for k, v in names.items() if len(v) > 1} == {
        "combine_kernel", "topk_stream_kernel", "sparse_bwd_kernel"}
    assert traffic.short_name(COMBINE_Q) == "combine_q"
    assert traffic.short_name(COMBINE_KV) == "combine_kv"
    role = "_ZN5elsaa17sparse_bwd_kernelIDF16bLi128ELi256ELi{}ELb0EEEvPKT_S3_S3_S3_PKfS5_S5_S5_PKiS7_iiiiS7_S7_fPS1_S8_S8_"
    assert traffic.short_name(role.format(1)) == "sparse_bwd"
    assert traffic.short_name(role.format(3)) == "sparse_bwd"
    assert traffic.short_name(role.format(2)) == "sparse_bwd_q"
    assert traffic.short_name("void elsaa::sparse_bwd_kernel<float, 64, 32, 2, false>(float const*)") == "sparse_bwd_q"


def test_summarize_calibrates_and_averages(tmp_path):
    kib = traffic.COPY_BYTES / 1024.0
    # Calibration runs: the copy reads half of what it moves as FETCH_SIZE and all of
    # it as WRITE_SIZE (the factors 2 and 1 seen on the GPU); a small unrelated
    # dispatch must not be taken for the copy.
    write_csv(tmp_path / "fc.csv", "FETCH_SIZE", [(1, "fill", 3.0), (2, "copy", kib / 4), (2, "copy", kib / 4)])
    write_csv(tmp_path / "wc.csv", "WRITE_SIZE", [(1, "fill", 1.0), (2, "copy", kib)])
    # Bench runs: two dispatches of the hash kernel (one counter row split over two
    # rows), one of a foreign kernel (ignored).
    hash_name = HASH
    write_csv(tmp_path / "fb.csv", "FETCH_SIZE",
              [(5, hash_name, 100.0), (5, hash_name, 20.0), (9, hash_name, 80.0), (7, "at::foo", 1e6)])
    write_csv(tmp_path / "wb.csv", "WRITE_SIZE", [(5, hash_name, 4.0), (9, hash_name, 6.0)])
    out = tmp_path / "t.json"
    traffic.summarize(str(out), str(tmp_path / "fb.csv"), str(tmp_path / "wb.csv"),
                      str(tmp_path / "fc.csv"), str(tmp_path / "wc.csv"))
    rec = json.load(open(out))
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert set(rec["kernels"]) == {"hash"}
    k = rec["kernels"]["hash"]
    assert k["fetch_kib_per_launch"] == 100.0  # (120 + 80) / 2 dispatches
    assert k["write_kib_per_launch"] == 5.0
    assert k["hbm_bytes_per_launch"] == round(100.0 * 1024 * 2 + 5.0 * 1024)
    assert rec["library_hash"] == traffic.library_hash()
