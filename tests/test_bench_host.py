"""Host-side logic of bench.py (no GPU): the one-GPU guard, the hot kernel's
roofline arithmetic, and the lookup of committed HBM-traffic figures, which
must be dropped once the kernel source no longer matches the hash they were
taken on."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")   # no JSON record


def test_layer_figures_roofline_arithmetic(bench):
    shape = synth.layer_shape(1)
    hot_ms, step_ms = 1.6, 1.8
    fig = bench.layer_figures(shape, step_ms, hot_ms)
    flops = 4.0 * shape.T * shape.H * shape.d * shape.I
    assert flops == pytest.approx(1.649e12, rel=1e-3)          # 4 T H d I for the Qwen3 layer
    roof = fig["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["peak"] == bench.PEAK_BF16_TFLOPS == 2500.0
    assert roof["achieved"] == pytest.approx(flops / (hot_ms * 1e-3) / 1e12)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    assert fig["tokens_per_s"] == pytest.approx(shape.T / (step_ms * 1e-3))
    assert fig["mfma_frac_whole_step"] == pytest.approx(flops / (step_ms * 1e-3) / 1e12 / 2500.0)
    # a, g, u read once in bf16, r and r_next in fp32
    stream = shape.T * (2 * (shape.H * shape.d + 2 * shape.I) + 8)
    assert fig["hot_stream_gbs"] == pytest.approx(stream / (hot_ms * 1e-3) / 1e9)


def test_fp32_layer_uses_the_fp32_peak(bench):
    shape = synth.layer_shape(1).with_dtype("f32")
    fig = bench.layer_figures(shape, 18.0, 17.0)
    assert fig["roofline"]["peak"] == bench.PEAK_FP32_TFLOPS == 157.3


def test_traffic_figures_follow_the_kernel_source(bench, tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    h = bench.hot_source_hash()
    path.write_text(json.dumps({
        "w-current:T=8": {"source_sha256_16": h, "bytes_per_launch": 1234.0},
        "w-stale:T=8": {"source_sha256_16": "0" * 16, "bytes_per_launch": 99.0},
    }))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_for("w-current:T=8") == 1234.0
    assert bench.traffic_for("w-stale:T=8") is None     # taken on another kernel source
    assert bench.traffic_for("w-absent:T=8") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("w-current:T=8") is None

