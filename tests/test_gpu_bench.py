"""bench.py's output contract on the GPU: one JSON line with the fields the
measurement needs, on small workloads (bench.py runs as a child process, one
at a time)."""
import json
import os
import subprocess
import sys

import pytest

from conftest import progress

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TOP_KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}
ROOF_KEYS = {"bound", "achieved", "peak", "unit", "frac", "traffic", "traffic_source"}


def _bench(*args):
    progress("bench.py " + " ".join(args))
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, "bench.py must print exactly one line, got %d" % len(lines)
    return json.loads(lines[0])


def _check_common(d, steps, warmup):
    assert TOP_KEYS <= set(d), TOP_KEYS - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and "scaling" not in d and d["data"] == "synthetic"
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert ROOF_KEYS <= set(roof), ROOF_KEYS - set(roof)
    assert roof["peak"] > 0 and roof["achieved"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert 0 < roof["frac"] < 1.2
    env = d["env"]
    assert env["hip"] and env["device"] and env["kernel_source_sha256_16"]
    src = roof["traffic_source"]
    assert "--pmc" in src["kind"] and src["kernel_source_sha256_16"]
    assert (roof["traffic"] is None) or src["matches_current_sources"]


def test_quantize_line_with_cpu_baselines():
    d = _bench("--workload", "bf16-4096x4096-rowscaled", "--steps", "3", "--warmup", "1")
    _check_common(d, 3, 1)
    assert d["unit"] == "GB/s" and d["roofline"]["bound"] == "hbm" and d["roofline"]["peak"] == 8000.0
    assert d["config"]["workload"] == "bf16-4096x4096-rowscaled"
    assert d["config"]["bytes_per_step"] == 4096 * 4096 * 2 + 4096 * 4096 + 4096 * 4096 // 32
    # steps run back to back, one launch per step: value equals the roofline's achieved rate
    assert abs(d["value"] - d["roofline"]["achieved"]) <= 0.01 * d["value"]
    pc = d["per_call"]
    assert pc["n"] == 20 and 0 < pc["min_us"] <= pc["median_us"]
    ref = d["copy_reference"]
    assert ref["GBps"] > 0 and abs(ref["value_over_copy"] - d["value"] / ref["GBps"]) < 1e-3
    for key in ("cpu_baseline", "cpu_baseline_all_cores"):
        cb = d[key]
        assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
        assert cb["host"]["model"]


def test_flushed_line():
    d = _bench("--workload", "bf16-4096x4096-rowscaled", "--cache", "flushed", "--steps", "3", "--warmup", "1",
               "--no-cpu-baseline")
    _check_common(d, 3, 1)
    assert d["config"]["cache"] == "flushed" and d["cpu_baseline"] is None


def test_matmul_line():
    # no --warmup: the matmul ops default to a long warm-up (the clock's settling time)
    d = _bench("--op", "matmul", "--mm", "512", "512", "512", "--steps", "2", "--no-cpu-baseline")
    _check_common(d, 2, 200)
    assert d["unit"] == "TFLOP/s" and d["roofline"]["bound"] == "mfma" and d["roofline"]["peak"] == 5000.0
    assert d["config"]["flops_per_step"] == 2.0 * 512 ** 3


def test_copy_calibration_line():
    progress("bench.py --copy-calibration")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--copy-calibration", "--steps", "2",
                        "--warmup", "1"], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["copy_bytes_read"] == d["copy_bytes_written"] == 2 << 30 and d["copy_GBps"] > 0


def test_vendor_gemm_line():
    """--vendor-gemm: the vendor's per-tensor FP8 product at small sizes, one
    JSON line with its time and rate (context only, not a bench line)."""
    d = _bench("--vendor-gemm", "--mm", "1024", "1024", "1024", "--steps", "3", "--warmup", "1")
    v = d["vendor_gemm"]
    assert (v["M"], v["N"], v["K"]) == (1024, 1024, 1024)
    assert v["us_per_call"] > 0 and v["TFLOPs"] > 0
    assert abs(v["TFLOPs"] - 2.0 * 1024 ** 3 / (v["us_per_call"] * 1e-6) / 1e12) < 0.05 * v["TFLOPs"] + 0.1
    assert d["steps"] == 3 and d["warmup"] == 1 and "metric" not in d
