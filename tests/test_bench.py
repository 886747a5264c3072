"""CPU: the benchmark's own arithmetic.  The per-kernel statistics, the
roofline object of the dominant kernel, the combined bound of the final
product and the counter-traffic lookup (which must go null once the kernel
source differs from the one the counters were taken on), plus the refusal of
more than one GPU.  No GPU and no library calls."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_stats_totals_and_rates():
    recs = [("gemm_symm_256", 1.0, 2e12, 1e9), ("gemm_symm_256", 1.0, 2e12, 1e9),
            ("row_score", 0.5, 0.0, 4e9)]
    kernels, by_shape = bench.kernel_stats(recs, steps=2)
    s = kernels["gemm_symm_256"]
    assert s["launches"] == 2 and s["avg_us"] == pytest.approx(1000.0)
    assert s["ms_per_step"] == pytest.approx(1.0)
    assert s["tflops"] == pytest.approx(2000.0)           # 4e12 flop in 2 ms
    assert s["frac_fp16_peak"] == pytest.approx(0.8)
    assert s["gbs"] == pytest.approx(1000.0)
    assert s["bound"] == "mfma" and s["frac_roofline"] == pytest.approx(0.8)
    r = kernels["row_score"]
    assert r["gbs"] == pytest.approx(8000.0) and r["bound"] == "hbm"
    assert r["frac_roofline"] == pytest.approx(1.0)
    assert by_shape[("gemm_symm_256", 2e12, 1e9)]["launches"] == 2


def test_roofline_is_the_dominant_kernel_by_time():
    recs = [("gemm_symm_256", 3.0, 3e12, 1e9), ("row_score", 1.0, 0.0, 5e9),
            ("gemm_poly_256", 2.0, 2e12, 1e9)]
    kernels, _ = bench.kernel_stats(recs, steps=1)
    r = bench.roofline_of(kernels, "no-such-workload")
    assert r["kernel"] == bench.KERNEL_SYMBOLS["gemm_symm_256"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(1000.0)          # 3e12 flop in 3 ms
    assert r["frac"] == pytest.approx(0.4)
    assert r["work_per_launch"] == pytest.approx(3e12)
    assert r["avg_launch_us"] == pytest.approx(3000.0)
    assert r["traffic"] is None                            # no counters for that workload


def test_roofline_of_a_streaming_kernel_is_hbm_bound():
    kernels, _ = bench.kernel_stats([("row_score", 2.0, 0.0, 1.2e10)], steps=1)
    r = bench.roofline_of(kernels, "x")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(6000.0) and r["frac"] == pytest.approx(0.75)
    assert r["work_per_launch"] == pytest.approx(1.2e10)


def test_multiply_back_takes_the_larger_of_its_two_bounds():
    recs = [("gemm_back_256", 1.0, 5e11, 6e9), ("gemm_back_256", 1.0, 5e11, 6e9),
            ("gemm_symm_256", 1.0, 1e12, 1e9)]
    kernels, _ = bench.kernel_stats(recs, steps=1)
    mb = bench.multiply_back_of(kernels)
    assert mb["tflops"] == pytest.approx(500.0) and mb["frac_fp16_peak"] == pytest.approx(0.2)
    assert mb["gbs"] == pytest.approx(6000.0) and mb["frac_hbm"] == pytest.approx(0.75)
    assert mb["bound"] == "hbm" and mb["frac_roofline"] == pytest.approx(0.75)
    assert bench.multiply_back_of({"gemm_symm_256": kernels["gemm_symm_256"]}) is None


def _tree(tmp_path, src_text, entry_hash):
    csrc = tmp_path / "orthogonalizing_optimizer_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "gemm_f16.hip").write_text(src_text)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(
        {"c4": {"gemm_symm_256": {"source_hash": entry_hash, "bytes_per_launch": 1234.0}}}))


def test_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    src = "// kernel source as profiled\n"
    good = hashlib.sha256(src.encode()).hexdigest()[:16]
    _tree(tmp_path, src, good)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash("gemm_symm_256") == good
    assert bench.load_traffic("gemm_symm_256", "c4") == 1234.0
    assert bench.load_traffic("gemm_symm_256", "c3") is None          # not profiled
    (tmp_path / "orthogonalizing_optimizer_amd" / "csrc" / "gemm_f16.hip").write_text(src + "x")
    assert bench.load_traffic("gemm_symm_256", "c4") is None          # source changed since


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
