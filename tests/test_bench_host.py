"""Host-side logic of bench.py (no GPU): the algorithmic byte counts that
price the kernels against the HBM roofline, the oracle's CPU legs, and the
refusal of more than one GPU."""

import json
import os
import subprocess
import sys

import pytest

import bench
from combine_topk_idx_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_large_workload_bytes_by_hand():
    w = W.WORKLOADS["large"]                    # T 16384, H 7168, k 8, int64 ids, MXFP4 dispatch, bf16 combine
    R = 124518
    b = bench.algorithmic_bytes(w, R)
    T, H, k, E = 16384, 7168, 8, 256
    assert b["layout"] == T * k * 8 + E * 8 + (E + 1) * 4 + T * k * 4 + R * 4
    assert b["dispatch"] == 2 * T * H + T * k * 4 + R * (H // 2 + H // 32)      # 3584 codes + 224 scale bytes
    assert b["combine"] == R * 2 * H + T * k * (8 + 4) + 2 * T * H                # bf16 rows, int64 ids, weights
    assert b["total"] == b["layout"] + b["dispatch"] + b["combine"]


@pytest.mark.parametrize("mode,row", [("none", (14336, 0)), ("int8_token", (7168, 4)), ("fp8_b128", (7168, 224)),
                                      ("fp8_b128_pow2", (7168, 224)), ("fp8_b128_ue8m0", (7168, 56)),
                                      ("mxfp8", (7168, 224)), ("mxfp4", (3584, 224))])
def test_row_bytes_match_the_receive_layout(mode, row):
    assert bench._row_bytes(mode, 7168) == row


def test_moe_bytes_and_flops_by_hand():
    w = W.MOE_WORKLOADS["moe_share"]            # H 7168, I 3072, 6 local experts
    R = 775
    a = bench.moe_algorithmic(w, R)
    H, I, E = 7168, 3072, 6
    assert a["bytes"]["gmm1"] == E * 2 * I * (H + H // 32) + R * (H + H // 32) + R * (I + I // 32)
    assert a["bytes"]["gmm2"] == E * H * (I + I // 32) + R * (I + I // 32) + R * 2 * H
    assert a["flops"]["gmm1"] == 2 * R * H * 2 * I and a["flops"]["gmm2"] == 2 * R * I * H


def test_cpu_legs_run_the_oracle_on_one_core():
    d = bench.cpu_baseline("small", 16)
    assert d["kind"] == "oracle" and d["cores"] == 1 and d["value"] > 0
    m = bench.cpu_baseline("moe_small", 8, moe=True)
    assert m["kind"] == "oracle" and m["cores"] == 1 and m["value"] > 0 and "GMM1" in m["sample"]


@pytest.mark.parametrize("extra", [[], ["--moe", "moe_share"]])
def test_more_than_one_gpu_is_refused(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", *extra],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_committed_counters_match_the_kernel_sources():
    """profiles/ holds rocprofv3 HBM byte counts for the measured kernels,
    stamped with a hash of the kernel sources they were taken on; bench.py
    reports them as `roofline.traffic` only while the sources still match.
    A kernel change must come with counters taken again."""
    large = bench._traffic("large")
    moe = bench._traffic("moe_share", bench.MOE_TRAFFIC_FILE, bench.MOE_KERNEL_SOURCES)
    assert large is not None, "profiles/combine_large_traffic.json was taken on other kernel sources"
    assert moe is not None, "profiles/gmm1_moe_share_traffic.json was taken on other kernel sources"
    with open(os.path.join(ROOT, "profiles", "combine_large_traffic.json")) as f:
        d = json.load(f)
    # counter bytes within a few percent of the algorithmic bytes: no wasted re-reads
    assert 1.0 <= d["traffic_over_alg"] < 1.05


def test_trace_summary_groups_by_kernel_and_grid(tmp_path):
    """--trace-summary --by-grid: one row per (kernel, workgroups x threads),
    durations from the start and end timestamps, longest total first."""
    import csv
    cols = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"]
    rows = [("KERNEL_DISPATCH", "void (anonymous namespace)::gather_kernel<8>(int const*)", 0, 5000, 128, 896 * 128),
            ("KERNEL_DISPATCH", "void (anonymous namespace)::gather_kernel<8>(int const*)", 0, 7000, 128, 896 * 128),
            ("KERNEL_DISPATCH", "void (anonymous namespace)::gather_kernel<8>(int const*)", 0, 340000, 128,
             114688 * 128),
            ("KERNEL_DISPATCH", "void empty_kernel()", 10, 1310, 128, 128)]
    (tmp_path / "run").mkdir()
    with open(tmp_path / "run" / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)
    lines = bench.trace_summary(str(tmp_path), by_grid=True).splitlines()
    assert lines[2] == "| `gather_kernel<8>` | 114688 x 128 | 1 | 340.00 | 340.00 | 340.00 | 340.00 |"
    assert lines[3] == "| `gather_kernel<8>` | 896 x 128 | 2 | 6.00 | 6.00 | 5.00 | 7.00 |"
    assert lines[4] == "| `empty_kernel` | 1 x 128 | 1 | 1.30 | 1.30 | 1.30 | 1.30 |"
