"""Host logic of bench.py (CPU only): the algorithmic bytes and flops behind the bench
line's GB/s and MFMA fraction, the one-GPU guard, and the traffic summary's staleness
check."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_default_workload():
    # Per query at N_c = 262,144, k = 512, W = 128, 64 + 64 heads: FP4 keys of 64 code and
    # 8 scale bytes, q_I (bf16) and w (fp32), 640 mixed rows of 576 bytes, q and out (bf16),
    # and the top-k indices the merge writes.
    keys = 262144 * 72
    q_i = 64 * 128 * 2 + 64 * 4
    rows = (512 + 128) * 576
    q_out = 2 * 64 * 512 * 2
    topk = 512 * 4
    b = bench.algorithmic_bytes(bench.WORKLOADS["csa_mixed_1m"])
    assert b["scan"] == 4 * (keys + q_i) == 75_564_032
    assert b["indexer"] == b["scan"] + 4 * topk
    assert b["attention"] == 4 * (rows + q_out)
    assert b["step"] == 4 * (keys + q_i + topk + rows + q_out) == 77_571_072


def test_algorithmic_bytes_of_the_reuse_stack_and_hca():
    w = bench.WORKLOADS["csa2_stack_fp4_1m"]
    b = bench.algorithmic_bytes(w)
    layer = 8 * ((512 + 128) * (256 + 32) + 2 * 64 * 512 * 2)  # FP4 rows: 256 code + 32 scale bytes
    assert b["attention"] == layer
    assert b["step"] == b["indexer"] + layer + 5 * (layer + 8 * 512 * 4)
    h = bench.algorithmic_bytes(bench.WORKLOADS["hca_bf16_1m"])
    assert h["step"] == 16 * ((8192 + 128) * 1024 + 2 * 64 * 512 * 2)
    assert h["scan"] == 0


def test_algorithmic_flops():
    # The scan's contraction: 2 flops per (head, channel, key); HCA: QK and PV, 2 each.
    assert bench.algorithmic_flops(bench.WORKLOADS["csa_mixed_1m"]) == 4 * 2 * 64 * 128 * 262144
    assert bench.algorithmic_flops(bench.WORKLOADS["csa_bf16_131k"]) == 32 * 2 * 64 * 128 * 32768
    assert bench.algorithmic_flops(bench.WORKLOADS["hca_bf16_1m"]) == 16 * 4 * 64 * 512 * (8192 + 128)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_null_once_the_kernel_sources_change(tmp_path, monkeypatch):
    src = tmp_path / "indexer.hip"
    src.write_text("// one version of the scan\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    summary = tmp_path / "traffic.txt"
    summary.write_text(f"kernel_sources_sha256: {bench.kernel_sources_sha256()}\n"
                       "traffic_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    assert bench.measured_traffic("csa_mixed_1m") == 123
    assert bench.measured_traffic("hca_bf16_1m") is None  # recorded for the default workload only
    src.write_text("// another version\n")
    assert bench.measured_traffic("csa_mixed_1m") is None
