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
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    s = bench.write_traffic_summary(str(f), str(w))
    assert s["copy_scale"]["fetch"] == pytest.approx(2.0) and s["copy_scale"]["write"] == pytest.approx(1.0)
    assert s["hbm_bytes_per_launch"] == round(1000.0 * 1024 * 2 + 200.0 * 1024)
    assert s["act_quant_hbm_bytes_per_launch"] == round(300.0 * 1024 * 2 + 100.0 * 1024)
    assert s["kernel_source_sha"] == bench.kernel_source_sha()
    assert json.load(open(out)) == s
    # the bench reports the stored figure only while the kernel source is unchanged
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus must be 1" in r.stderr
