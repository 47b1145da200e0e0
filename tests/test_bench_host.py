"""bench.py's host-side logic, on the CPU: the one-GPU contract, the roofline
arithmetic and the rule that a committed HBM-traffic figure is reported only
for the GEMM source it was measured on."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)        # defines functions only; the run is behind __main__
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""        # no JSON line


def test_roofline_fractions(bench):
    # 1250 TFLOP/s on the exact inner product, 2000 MHz measured
    r = bench.mfma_roofline(1250.0, 0.7, 9.62e11, 2000.0, "k", True)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 5000.0
    assert r["frac"] == pytest.approx(0.25)
    assert r["f16_ceiling"]["frac"] == pytest.approx(0.5)
    assert r["peak_at_measured_clock"] == pytest.approx(5000.0 * 2000.0 / 2400.0, abs=0.05)
    assert r["frac_at_measured_clock"] == pytest.approx(0.3, abs=1e-4)
    assert r["f16_ceiling"]["frac_at_measured_clock"] == pytest.approx(0.6, abs=1e-4)
    assert r["traffic"] is None
    # the fast inner product has no f16 ceiling; no clock given, no clock fields
    r = bench.mfma_roofline(2500.0, 0.4, 9.62e11, None, "k", False)
    assert r["frac"] == pytest.approx(0.5)
    assert "f16_ceiling" not in r and "clock_mhz_measured" not in r


def test_traffic_figure_needs_the_measured_gemm_source(bench, tmp_path, monkeypatch):
    good = bench.gemm_source_hash()
    f = tmp_path / "traffic.md"
    f.write_text(f"x\n```\ngemm_source_sha256: {good}\ntraffic_bytes_per_launch: 123456789\n```\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.gemm_traffic() == 123456789.0
    f.write_text(f"gemm_source_sha256: {'0' * 64}\ntraffic_bytes_per_launch: 123456789\n")
    assert bench.gemm_traffic() is None          # counters taken on another source
    f.write_text(f"gemm_source_sha256: {good}\n")
    assert bench.gemm_traffic() is None          # no figure
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.md"))
    assert bench.gemm_traffic() is None


def test_cpu_model_names_the_host(bench):
    name = bench.cpu_model()
    assert isinstance(name, str) and name
