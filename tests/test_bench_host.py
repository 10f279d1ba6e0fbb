"""Host logic of bench.py (CPU): the speedup chart's table and image, the
command-line checks that run before any GPU work."""
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMMS = [("qkv", "fprop", 256, 768, 512), ("qkv", "dgrad", 256, 512, 768), ("mlp_up", "wgrad", 512, 1024, 256)]


def _fake(ms):
    """A runner with three GEMMs and per-GEMM timings ms[(recipe, layer, pass)]."""
    runner = types.SimpleNamespace(gemms=GEMMS)
    per = {k: {"auto": [v * 1.1, v, v * 0.9]} for k, v in ms.items()}     # median v
    pre = {k: (v / 2, v / 3) for k, v in ms.items()}                       # (median, min)
    return runner, per, pre


def test_speedup_table_autocast_and_prequant():
    ms = {}
    for (n, p, *_) in GEMMS:
        ms[("bf16", n, p)] = 2.0
        ms[("fp8_current", n, p)] = 1.0
        ms[("nvfp4", n, p)] = 4.0
    runner, per, pre = _fake(ms)
    labels, tab, kind = bench.speedup_table(runner, ["bf16", "fp8_current", "nvfp4"], per)
    assert kind == "speedup" and labels == ["qkv.fprop", "qkv.dgrad", "mlp_up.wgrad"]
    assert set(tab) == {"fp8_current", "nvfp4"}
    assert np.allclose(tab["fp8_current"], 2.0) and np.allclose(tab["nvfp4"], 0.5)
    # pre-quantized: the medians of `pre` (ms / 2 for every recipe: same ratios)
    _, tab_p, _ = bench.speedup_table(runner, ["bf16", "fp8_current"], per, pre)
    assert np.allclose(tab_p["fp8_current"], 2.0)


def test_speedup_table_without_bf16_is_tflops():
    ms = {("fp8_current", n, p): 0.5 for (n, p, *_) in GEMMS}
    runner, per, _ = _fake(ms)
    _, tab, kind = bench.speedup_table(runner, ["fp8_current"], per)
    assert kind == "TFLOP/s"
    want = [2.0 * M * N * K / 0.5e-3 / 1e12 for (_, _, M, N, K) in GEMMS]
    assert np.allclose(tab["fp8_current"], want)


def test_speedup_plot_writes_a_png(tmp_path):
    ms = {(r, n, p): v for (n, p, *_) in GEMMS for r, v in (("bf16", 2.0), ("mxfp8", 1.2))}
    runner, per, _ = _fake(ms)
    out = bench.write_speedup_plot(str(tmp_path / "charts" / "speedup.png"), runner, ["bf16", "mxfp8"], per, None,
                                   "test")
    with open(out, "rb") as f:
        assert f.read(8) == b"\x89PNG\r\n\x1a\n"


def test_models_carry_their_layer_counts():
    assert bench.MODELS["codonfm"]["num_layers"] == 24
    assert bench.MODELS["llama3_8b"]["num_layers"] == 32


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
