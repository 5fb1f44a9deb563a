"""Host-side logic of bench.py (no GPU needed): the byte counts behind the
roofline, the source-digest gate on recorded traffic, the one-GPU refusal
and the CPU-baseline records."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Per-configuration byte counts as the workload table states them (input,
# data and logical scale bytes), for the five quantize configurations.
SIZE_TABLE = [
    (128, 512, "e4m3fn", 131072, 65536, 2048),
    (4096, 4096, "e4m3fn", 33554432, 16777216, 524288),
    (8192, 14336, "e5m2", 234881024, 117440512, 3670016),
    (16384, 8192, "e2m1", 268435456, 67108864, 4194304),
    (131072, 8192, "e4m3fn", 2147483648, 1073741824, 33554432),
]


@pytest.mark.parametrize("P,F,out,in_b,data_b,scale_b", SIZE_TABLE)
def test_algorithmic_bytes_match_the_size_table(P, F, out, in_b, data_b, scale_b):
    assert bench.algorithmic_bytes(P, F, out) == in_b + data_b + scale_b


def test_algorithmic_bytes_per_element():
    # 2 + 1 + 1/32 for FP8 and 2 + 1/2 + 1/32 for FP4
    assert bench.algorithmic_bytes(1024, 1024, "e4m3fn") / (1024 * 1024) == 3.03125
    assert bench.algorithmic_bytes(1024, 1024, "e2m1") / (1024 * 1024) == 2.53125


def test_dequant_bytes():
    n = 4096 * 8192
    assert bench.dequant_bytes(4096, 8192, "e4m3fn", "bf16") == n + n // 32 + 2 * n
    assert bench.dequant_bytes(4096, 8192, "e2m1", "f32") == n // 2 + n // 32 + 4 * n


def _summary(digest: str, nbytes: float) -> str:
    return "header\n\nkernel_source_sha256_16: %s\n\nhbm_bytes_per_launch: %.0f\n" % (digest, nbytes)


def test_recorded_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    tag = "quantize_wl_e4m3fn"
    path = tmp_path / ("%s_hbm_traffic.txt" % tag)
    t, src = bench.recorded_traffic("wl", "e4m3fn")
    assert t is None and src["file"] is None                            # no summary
    path.write_text(_summary(bench.kernel_source_digest("quantize"), 3254863572))
    t, src = bench.recorded_traffic("wl", "e4m3fn")
    assert t == 3254863572.0 and src["matches_current_sources"]          # current sources
    assert src["kernel_source_sha256_16"] == bench.kernel_source_digest("quantize")
    assert src["file"].endswith("quantize_wl_e4m3fn_hbm_traffic.txt") and "--pmc" in src["kind"]
    path.write_text(_summary("0123456789abcdef", 3254863572))
    t, src = bench.recorded_traffic("wl", "e4m3fn")
    assert t is None and not src["matches_current_sources"]              # stale sources
    path.write_text("kernel_source_sha256_16: %s\n" % bench.kernel_source_digest("quantize"))
    assert bench.recorded_traffic("wl", "e4m3fn")[0] is None             # no byte count


def test_recorded_traffic_digest_is_per_op(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "dequantize_wl_e4m3fn_bf16_hbm_traffic.txt").write_text(
        _summary(bench.kernel_source_digest("quantize"), 1.0))
    # a dequantize summary carrying the quantize digest is not accepted
    if bench.kernel_source_digest("quantize") != bench.kernel_source_digest("dequantize"):
        assert bench.recorded_traffic("wl", "e4m3fn", "dequantize", "bf16")[0] is None


def test_bench_line_has_no_scaling_key():
    """One GPU: no weak/strong scaling claim on the line."""
    text = open(os.path.join(ROOT, "bench.py")).read()
    assert '"scaling"' not in text


def test_every_kernel_source_exists():
    for op, files in bench.KERNEL_SOURCES.items():
        for rel in files:
            assert os.path.exists(os.path.join(ROOT, rel)), (op, rel)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bad_step_counts_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU exit")
@pytest.mark.parametrize("mode", [[], ["--vendor-gemm"]])
def test_no_gpu_fails_loudly(mode):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "0"] + mode,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 1
    assert "no GPU" in r.stderr
    assert r.stdout == ""


def test_default_warmup():
    assert bench.default_warmup("quantize", None) == 5
    assert bench.default_warmup("dequantize", None) == 5
    assert bench.default_warmup("quantize_axis", None) == 5
    assert bench.default_warmup("matmul", None) == bench.MATMUL_WARMUP == 200
    assert bench.default_warmup("matmul_quantize", None) == 200
    assert bench.default_warmup("matmul", 3) == 3 and bench.default_warmup("quantize", 0) == 0


def test_host_cpu_record():
    h = bench.host_cpu()
    assert isinstance(h["model"], str) and h["model"]
    assert 1 <= h["usable_cpus"] <= h["logical_cpus"]


def _host_input(P, F, seed):
    bits = workloads.random_bits(P, F, "bf16", seed=seed, specials=False)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def test_cpu_baseline_record():
    xt = _host_input(256, 512, 3)
    rec = bench.cpu_baseline(xt, "e4m3fn", "bf16", budget_s=0.5, slab_rows=64)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["unit"] == "GB/s"
    assert rec["value"] > 0
    assert "of 256 rows" in rec["sample"]
    json.dumps(rec)


def test_cpu_baseline_all_cores_record():
    xt = _host_input(256, 512, 4)
    rec = bench.cpu_baseline_all_cores(xt, "e2m1", "bf16", max_threads=4)
    assert rec["kind"] == "oracle" and rec["value"] > 0
    assert rec["cores"] == min(4, os.cpu_count() or 1, 256 // 32)
    json.dumps(rec)
