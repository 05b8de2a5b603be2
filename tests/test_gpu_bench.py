"""bench.py end to end on the GPU, on the smallest workload (one 1M-parameter
tensor, 8-bit moments): the JSON line carries the fields the benchmark
reports (with the stream probe's ceiling), with values consistent with each
other, and the stream-probe mode reports every residency cap."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def _run(*args):
    print("bench.py", *args, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def test_bench_line_on_a_small_workload():
    d = _run("--config", "single_q8", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "Gparams/s" and d["value"] > 0 and d["higher_is_better"] is True
    cfg = d["config"]
    assert cfg["workload"] == "single_q8" and cfg["params"] == 1 << 20 and cfg["storage"] == "q8"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    # value (Gparams/s) and achieved (GB/s) come from the same step time
    sec = d["ms_per_step"] / 1e3
    assert abs(d["value"] - cfg["params"] / sec / 1e9) <= 1e-3 * d["value"] + 1e-3
    assert abs(roof["achieved"] - roof["algorithmic_bytes_per_launch"] / sec / 1e9) <= 0.1 + 1e-3 * roof["achieved"]
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # the stream probe's ceiling on the same blocks, and the step's fraction of it
    ceil = roof["pattern_ceiling"]
    assert ceil["best_cap"] in (2, 3, 4, 5, 6, 8) and 0 < ceil["frac"] < 1.5
    assert abs(ceil["step_over_ceiling"] - roof["frac"] / ceil["frac"]) < 1e-3


def test_stream_probe_mode_on_a_small_workload():
    d = _run("--stream-probe", "--config", "single_q8", "--steps", "2", "--warmup", "1")
    (rec,) = d["stream_probe"]
    assert rec["workload"] == "single_q8" and rec["blocks"] == 512
    assert rec["bytes_per_launch"] == 512 * (2048 * (8 + 4 + 2 + 2) + 16)
    assert set(rec["resident_per_cu"]) == {"2", "3", "4", "5", "6", "8"}
    for v in rec["resident_per_cu"].values():
        assert v["ms_per_launch"] > 0 and 0 < v["frac"] < 1.5
