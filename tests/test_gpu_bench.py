"""bench.py end to end on the tiny layer: every mode prints one JSON line with
the fields the benchmark contract names, and its numbers hang together."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*extra):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny", "--steps", "4", "--warmup", "2",
           "--no-cpu", "--no-ceiling", *extra]
    print(" ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


@pytest.mark.parametrize("extra", [(), ("--staged",), ("--pad-multiple", "16"), ("--graph",),
                                   ("--graph", "--graph-steps", "2"), ("--events", "all"),
                                   ("--gather-mode", "2"), ("--warm",)])
def test_bench_line(extra):
    d = run_bench(*extra)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 2 and d["unit"] == "GB/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    cfg = d["config"]
    # value is the step's algorithmic bytes over the wall time per step
    assert abs(d["value"] - cfg["bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"] + 0.01
    if "--graph" in extra:
        assert d["roofline"] is None          # kernel events are for eager launches
        per_graph = extra[-1] if "--graph-steps" in extra else "1"
        assert f"{per_graph} step(s) per graph" in cfg["timing"]
        assert cfg["step_us"]["n"] == 4 // int(per_graph)
    else:
        r = d["roofline"]
        assert r["bound"] == "hbm" and r["peak"] == 8000.0 and 0 < r["frac"] < 1
        assert abs(r["achieved"] - r["algorithmic_bytes_per_launch"] / (r["avg_launch_us"] * 1e-6) / 1e9) \
            <= 0.01 * r["achieved"] + 0.1
