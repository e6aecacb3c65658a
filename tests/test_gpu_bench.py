"""bench.py's output contract on the GPU: one JSON line with the fields the benchmark
contract names, consistent with each other (a short run: few steps, no extras)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "5",
                        "--no-extras", "--cpu-rows", "64"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # the default workload is the largest one; value is the GEMM's flops per step time
    assert d["config"]["workload"].startswith("outlier")
    assert (d["config"]["M"], d["config"]["N"], d["config"]["K"], d["config"]["out"]) == (16384, 7168, 7168, "f32")
    flops = 2.0 * 16384 * 7168 * 7168
    assert d["value"] == pytest.approx(flops / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-3)
    assert d["pct_of_fp8_peak"] == pytest.approx(100.0 * d["value"] / 5000.0, rel=1e-3)
    rf = d["roofline"]
    # fp32 output: the default exact-slice contraction, priced against the f16 matrix unit
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    med, p10, p90 = rf["launch_us_median_p10_p90"]
    assert 0 < p10 <= med <= p90
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    assert rf["achieved"] == pytest.approx(rf["algorithmic_flops_per_launch"] / (rf["avg_launch_us"] * 1e-6) / 1e12,
                                           rel=1e-3)
    assert rf["traffic"] is None or rf["traffic"] > 0
    assert rf["mfma_busy_frac"] is None or 0 < rf["mfma_busy_frac"] < 1
    aq = d["act_quant"]
    assert aq["hbm_copy_reference"]["gbs"] > 0 and 0 < aq["back_to_back_frac_of_copy"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    assert cb["host"]["nproc"] >= 1 and cb["host"]["omp_threads"] == cb["cores"]
    assert cb["gpu_codes_match_oracle_on_sample"] is True
    assert cb["gpu_scales_match_oracle_on_sample"] is True
