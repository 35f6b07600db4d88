"""Host-side logic of bench.py that needs no GPU: the one-GPU guard and the
rule that the recorded HBM traffic is reported only for the GEMM sources it
was measured with."""
import hashlib
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _sources_sha(bench):
    h = hashlib.sha256()
    for name in bench.TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "transformer_encoder_bf16_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


@pytest.mark.parametrize("n", [0, 2, 8])
def test_bench_refuses_anything_but_one_gpu(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a refused run


def test_traffic_needs_the_measured_sources(bench, monkeypatch):
    t = dict(bench.TRAFFIC)
    expect = round(t["fetch_kib"] * 1024 / t["fetch_per_byte"] +
                   t["write_kib"] * 1024 / t["write_per_byte"])
    monkeypatch.setitem(bench.TRAFFIC, "sources_sha256", _sources_sha(bench))
    assert bench.measured_traffic(t["op"], t["workload"]) == expect
    # another op class or workload: no figure
    assert bench.measured_traffic("qkv_gemm", t["workload"]) is None
    assert bench.measured_traffic(t["op"], "short_1") is None
    # sources that differ from the measured ones: no figure
    monkeypatch.setitem(bench.TRAFFIC, "sources_sha256", "0" * 64)
    assert bench.measured_traffic(t["op"], t["workload"]) is None


def test_traffic_calibration_factors_are_the_copy_kernel_ones(bench):
    # a plain device copy of N bytes reads FETCH_SIZE N/2 and WRITE_SIZE N
    # (same units; the calibration recorded with the counters)
    assert bench.TRAFFIC["fetch_per_byte"] == pytest.approx(0.5)
    assert bench.TRAFFIC["write_per_byte"] == pytest.approx(1.0)
    # the recorded traffic is at least the kernel's algorithmic bytes
    # (A, the W rows read and the GeGLU output at T = 4050, H = 1024, F = 2624)
    T, H, F = 4050, 1024, 2624
    algorithmic = (T * H + 2 * F * H + T * F) * 2
    t = bench.TRAFFIC
    measured = t["fetch_kib"] * 1024 / t["fetch_per_byte"] + t["write_kib"] * 1024 / t["write_per_byte"]
    assert measured >= algorithmic
    # the writes are the GeGLU output exactly (rows live at T = 4050)
    assert t["write_kib"] * 1024 / t["write_per_byte"] == pytest.approx(T * F * 2, rel=1e-3)
