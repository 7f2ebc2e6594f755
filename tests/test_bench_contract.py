"""The benchmark's command line and its one-line JSON report.

CPU: more than one GPU is refused before anything touches a device.  GPU: a
short run on the c2 workload prints exactly one JSON line with the fields the
report promises, a roofline whose fraction is its achieved rate over the
peak, and the CPU oracle baseline beside it.
"""
import contextlib
import io
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_json_line():
    sys.path.insert(0, ROOT)
    import bench
    argv = sys.argv
    out = io.StringIO()
    try:
        sys.argv = ["bench.py", "--config", "c2", "--steps", "2", "--warmup", "1"]
        with contextlib.redirect_stdout(out):
            bench.main()
    finally:
        sys.argv = argv
    lines = [l for l in out.getvalue().splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"].startswith("c2:")
    assert "model" not in d["config"]
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2516.6
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
