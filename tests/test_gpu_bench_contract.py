"""bench.py's output line on the GPU: one JSON object with the fields the
result is read from, consistent with each other.  A short run (3 timed steps,
no extras, no CPU leg) in a child process."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_consistent_json_line():
    print("bench contract: short bench run", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", "--no-extras"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["data"] == "synthetic" and "workload" in d["config"]
    B = d["config"]["batch"]
    # value: attention tokens per second of the timed steps
    assert abs(d["value"] - B / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    # achieved = algorithmic bytes / mean launch time
    want = roof["algorithmic_bytes_per_launch"] / (roof["launch_ms_mean"] * 1e-3) / 1e9
    assert abs(roof["achieved"] - want) <= 1e-6 * want
    assert 0.3 < roof["frac"] < 1.0
    # HBM counters of the current sources: within 1% of the algorithmic bytes
    if roof["traffic"] is not None:
        assert abs(roof["traffic"] / roof["algorithmic_bytes_per_launch"] - 1.0) < 0.01
