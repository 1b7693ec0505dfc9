"""Host logic of bench.py, on the CPU: the one-GPU guard, the gating of the traffic figure on
the kernel source it was measured on, and the choice of roofline (MFMA peak or HBM bandwidth)
from Linear1's arithmetic intensity."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synth import CONFIGS  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_code_hash_ignores_comments_and_whitespace():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* twice */ }"
    b = "int f(int x){return 2*x;}"
    assert bench.code_hash(a) == bench.code_hash(b)
    assert bench.code_hash(a) != bench.code_hash("int f(int x){return 3*x;}")


def test_traffic_only_for_the_kernel_it_was_measured_on(monkeypatch):
    path = os.path.join(ROOT, "profiles", "linear1_c2_pmc.md")
    if not os.path.exists(path):
        pytest.skip("no committed counter summary")
    text = open(path).read()
    recorded = text.split("gemm_source_sha256_16:")[1].split()[0]
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: recorded)
    t = bench.load_traffic("c2")
    assert t is not None and t > 0
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("c2") is None
    assert bench.load_traffic("no_such_workload") is None


def _w1_bytes(c):
    return c.E * (2 * c.I * c.H // 2 + 2 * c.I * c.H // 32)   # FP4 codes + UE8M0 scales


@pytest.mark.parametrize("name,bound", [("c1", "hbm"), ("c2", "mfma"), ("c3", "mfma"), ("c4", "mfma")])
def test_roofline_bound_follows_arithmetic_intensity(name, bound):
    c = CONFIGS[name]
    r = bench.linear1_roofline(c.T, c.k, c.H, c.I, c.E, c.E, _w1_bytes(c), 1.0, None)
    assert r["bound"] == bound
    P = c.T * c.k
    if bound == "mfma":
        assert r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_TFLOPS
        assert r["achieved"] == pytest.approx(4.0 * P * c.H * c.I / 1e-3 / 1e12, rel=1e-4)
    else:
        nbytes = _w1_bytes(c) + P * (c.H + c.I + c.I // 128)
        assert r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
        assert r["achieved"] == pytest.approx(nbytes / 1e-3 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)


def test_roofline_counts_only_experts_that_receive_rows():
    c = CONFIGS["c1"]
    full = bench.linear1_roofline(c.T, c.k, c.H, c.I, c.E, c.E, _w1_bytes(c), 1.0, None)
    half = bench.linear1_roofline(c.T, c.k, c.H, c.I, c.E, c.E // 2, _w1_bytes(c), 1.0, None)
    assert half["achieved"] < full["achieved"]
    P = c.T * c.k
    expect = _w1_bytes(c) / 2 + P * (c.H + c.I + c.I // 128)
    assert half["achieved"] == pytest.approx(expect / 1e-3 / 1e9, rel=1e-4)


def test_host_cpu_description():
    model, phys, logical, usable = bench.host_cpu()
    assert isinstance(model, str) and model
    assert logical >= 1 and 1 <= usable <= logical
    assert phys is None or 1 <= phys <= logical


def test_cpu_baseline_times_the_cpp_oracle():
    """The baseline leg runs the plain C++ oracle on the first tokens of a batch and reports
    its rate, the threads it used and the host's CPU (tiny workload, a few tokens)."""
    from synth import make_inputs
    cfg = CONFIGS["c0"]
    host = make_inputs(cfg, seed=0).numpy()
    cb = bench.cpu_baseline(host, cfg, 8)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["cpu_model"]
    assert "first 8 tokens" in cb["sample"] and "C++" in cb["sample"]
