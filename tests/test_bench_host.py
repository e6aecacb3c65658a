"""Host-side pieces of bench.py (no GPU): the counter parsing behind roofline.traffic, the
traffic summary's scaling and source hash, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM = "void fp8q::block_gemm_kernel<128, 192, 8, 2, 3, 1, 0, 0, 0>(fp8q::GemmArgs)"
GROUPED = "void fp8q::block_gemm_kernel<128, 256, 8, 2, 3, 1, 0, 1, 0>(fp8q::GemmArgs)"
ROWWISE = "void fp8q::block_gemm_kernel<128, 192, 8, 2, 3, 0, 1, 0, 1>(fp8q::GemmArgs)"
AQ = "fp8q::act_quant_kernel(unsigned int __vector(4) const*, unsigned int __vector(2)*, float*, long)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(...)"


def _write_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value); a counter is reported in several rows per
    dispatch (one per hardware instance), which the parser sums."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, k, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": "OTHER", "Counter_Value": 1e9})


def test_per_dispatch_sums_instances_and_averages_dispatches(tmp_path):
    p = tmp_path / "c.csv"
    rows = [(1, GEMM, 100.0), (1, GEMM, 50.0),        # dispatch 1: 150
            (2, GEMM, 170.0),                         # dispatch 2: 170
            (3, GROUPED, 9999.0), (4, ROWWISE, 8888.0),   # not the plain GEMM
            (5, AQ, 30.0), (5, AQ, 10.0), (6, AQ, 60.0),
            (7, COPY, 2048.0)]
    _write_csv(p, "FETCH_SIZE", rows)
    got = bench._per_dispatch(str(p), "FETCH_SIZE")
    assert got == {"gemm": 160.0, "act_quant": 50.0, "copy": 2048.0}


def test_traffic_summary_scaling_and_hash(tmp_path, monkeypatch):
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    kib = bench.COPY_BYTES / 1024.0
    # the counter reports half the copy's bytes read and all of its bytes written
    _write_csv(f, "FETCH_SIZE", [(1, COPY, kib / 2), (2, GEMM, 1000.0), (3, AQ, 300.0)])
    _write_csv(w, "WRITE_SIZE", [(1, COPY, kib), (2, GEMM, 200.0), (3, AQ, 100.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda wl: str(out))
    s = bench.write_traffic_summary(str(f), str(w), "kv_down")
    assert s["workload"].startswith("kv_down 4096x576x7168")
    assert s["copy_scale"]["fetch"] == pytest.approx(2.0) and s["copy_scale"]["write"] == pytest.approx(1.0)
    assert s["hbm_bytes_per_launch"] == round(1000.0 * 1024 * 2 + 200.0 * 1024)
    assert s["act_quant_hbm_bytes_per_launch"] == round(300.0 * 1024 * 2 + 100.0 * 1024)
    assert s["kernel_source_sha"] == bench.kernel_source_sha()
    assert json.load(open(out)) == s
    # the bench reports the stored figure only while the kernel source is unchanged
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.measured_traffic("kv_down") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus must be 1" in r.stderr


def test_mfma_busy_summary(tmp_path, monkeypatch):
    """MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs * SIMDs), per GEMM
    dispatch (rocprofv3's MfmaUtil); other kernels are ignored; the stored figure is used only
    while the kernel source is unchanged."""
    p = tmp_path / "m.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, busy, gui in ((1, 512000.0, 8000.0), (2, 256000.0, 8000.0)):
            # eight XCD instances of the GUI counter, busy split over two SE rows
            for _ in range(8):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": GEMM, "Counter_Name": "GRBM_GUI_ACTIVE",
                            "Counter_Value": gui / 8})
            for _ in range(2):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": GEMM, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                            "Counter_Value": busy / 2})
        w.writerow({"Dispatch_Id": 3, "Kernel_Name": AQ, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                    "Counter_Value": 1e12})
    out = tmp_path / "mfma.json"
    monkeypatch.setattr(bench, "mfma_file", lambda wl: str(out))
    s = bench.write_mfma_summary(str(p), "outlier")
    assert s["workload"].startswith("outlier 16384x7168x7168")
    # mean busy 384000 over 1000 cycles x 1024 SIMDs
    assert s["kernel_cycles"] == pytest.approx(1000.0)
    assert s["mfma_busy_frac"] == pytest.approx(384000.0 / (1000.0 * 1024), abs=1e-4)
    assert bench.measured_mfma_busy("outlier") == s["mfma_busy_frac"]
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "f" * 16)
    assert bench.measured_mfma_busy("outlier") is None


def test_bench_rejects_unknown_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "no_such_shape"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "unknown workload" in r.stderr


def test_counter_files_are_per_workload():
    assert bench.traffic_file("kv_up").endswith(os.path.join("profiles", "gemm_kv_up_traffic.json"))
    assert bench.mfma_file("outlier").endswith(os.path.join("profiles", "gemm_outlier_mfma_busy.json"))


def test_cpu_sample_is_bounded():
    """The CPU baseline's row sample is about 1e11 multiply-adds (a few seconds of the oracle on
    16 host cores), a multiple of 64 rows, never more than the workload's rows."""
    import synth
    for wl in synth.WORKLOADS.values():
        r = bench.cpu_sample_rows(wl.M, wl.N, wl.K)
        assert 1 <= r <= wl.M
        assert r == wl.M or r * wl.N * wl.K <= bench.CPU_SAMPLE_MACS
        assert r == wl.M or r % 64 == 0
    assert bench.cpu_sample_rows(16384, 7168, 7168) == 1920


def test_host_cpu_fields():
    h = bench.host_cpu()
    assert h["nproc"] >= 1 and h["cpu_count"] >= h["nproc"]


def test_committed_counters_are_of_the_current_gemm_source():
    """Every committed counter summary (the MFMA-busy and traffic figures bench.py reports)
    was taken on the GEMM source as it is now: its stored hash is the current one, and so is
    the hash the markdown summaries of the same collection name. A change to the GEMM source
    without a new collection fails here instead of leaving bench.py to report nulls."""
    sha = bench.kernel_source_sha()
    for wl in ("outlier", "kv_up", "kv_down", "q_down"):
        for path in (bench.traffic_file(wl), bench.mfma_file(wl)):
            with open(path) as f:
                assert json.load(f)["kernel_source_sha"] == sha, path
    for name in ("gemm_workloads_counters.md", "gemm_workloads_kernel_trace.md", "bench_outlier_kernel_trace.md",
                 "gemm_outlier_issue_counters.md"):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            assert f"`{sha}`" in f.read(), name
