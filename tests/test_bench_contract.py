"""bench.py's command-line contract: one GPU only (checked without a GPU), and
on a GPU one JSON line with the fields the measurement needs."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_json_line():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5",
                        "--warmup", "2", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"].startswith("decode_bf16_T16_E64_H4096_I1536_k8")
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    # the FFN launches alone, and how many samples each figure rests on (a short
    # run still brackets FC1 on every step)
    ffn = d["ffn_roofline"]
    assert ffn["bound"] == "hbm" and 0 < ffn["frac"] < 1 and ffn["ffn_ms"] > 0
    assert d["samples"]["fc1_events"] == 5 and d["samples"]["step_intervals"] == 4
    assert d["samples"]["ffn_only"] == 5 and roof["samples"] == 5


@pytest.mark.gpu
@pytest.mark.parametrize("args,suffix", [
    (["--config", "3", "--weight-only"], "_w8a16"),
    (["--config", "3", "--block-fp8"], "_block128"),
    (["--config", "2", "--small-path"], "_small_path"),
    (["--config", "3", "--single-launch"], "_single_launch"),
    (["--config", "5", "--fp8"], "prefill_fp8_"),
])
def test_bench_modes(args, suffix):
    """Every measurement mode of the benchmark prints one line naming its workload."""
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline", *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    wl = d["config"]["workload"]
    assert wl.endswith(suffix) or wl.startswith(suffix), wl
    assert d["value"] > 0 and d["roofline"]["achieved"] > 0 and d["cpu_baseline"] is None
    if wl.startswith("prefill"):
        # the bound named is the longer of the MFMA and the HBM time, the other
        # fraction rides along
        roof = d["roofline"]
        bms = roof["bound_ms"]
        assert roof["bound"] == max(bms, key=bms.get)
        other = "mfma" if roof["bound"] == "hbm" else "hbm"
        assert 0 < roof[other]["frac"] < 1 and 0 < roof["frac"] < 1
