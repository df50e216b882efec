"""bench.py on the GPU: short runs print the one JSON line the contract asks for.

Two short parts of the benchmark, each in its own process: the LL sweep (the
line's value) and the HB prefill (its roofline).  Every field the contract
names must be there with the right type, every timed configuration must have
passed its oracle check, and the roofline must be consistent with itself.
"""
import json
import subprocess
import sys
from pathlib import Path

import pytest
import torch

from gpu_util import note

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parent.parent


def _run(*args):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    note(f"bench.py {' '.join(args)}")
    res = subprocess.run([sys.executable, "-u", str(ROOT / "bench.py"), *args],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [l for l in res.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    return json.loads(lines[0])


def _contract(line, steps, warmup):
    assert isinstance(line["metric"], str) and line["metric"]
    assert line["unit"] == "us" and line["n_gpus"] == 1
    assert line["steps"] == steps and line["warmup"] == warmup
    assert line["higher_is_better"] is False and line["scaling"] in ("weak", "strong")
    assert line["vs_baseline"] is None and line["dtype"] == "bf16"
    assert line["data"] == "synthetic" and isinstance(line["config"]["workload"], str)


def test_sweep_line():
    line = _run("--only", "sweep", "--steps", "2", "--warmup", "1", "--no-cpu", "--no-tune")
    _contract(line, 2, 1)
    rows = line["ll_sweep"]
    assert [r["bytes_per_rank"] for r in rows] == [2 << k for k in range(10, 20)]
    assert all(r["ll_parity"] and r["hb_parity"] for r in rows)
    assert line["value"] == pytest.approx(sum(r["ll_us"] for r in rows) / len(rows), abs=2e-3)
    # the floor is a one-workgroup call: below the slowest LL call on any machine
    assert 0 < line["graph_floor_us"] < max(r["ll_us"] for r in rows)
    assert line["ll_mean_above_floor_us"] == pytest.approx(
        line["value"] - line["graph_floor_us"], abs=2e-3)
    assert line["ms_per_step"] == pytest.approx(sum(r["ll_us"] for r in rows) * 10 / 1000,
                                                abs=1e-3)


def test_prefill_roofline():
    line = _run("--only", "prefill", "--steps", "3", "--warmup", "1", "--no-cpu", "--no-tune")
    _contract(line, 3, 1)
    assert line["hb_prefill"]["parity"] is True
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["bytes_per_launch"] == 2 << 30
    assert roof["achieved"] == pytest.approx(
        roof["bytes_per_launch"] / (roof["us_per_launch"] * 1e-6) / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    # traffic is the committed counter reading (checked against the sources on the CPU)
    assert roof["traffic"] is None or abs(roof["traffic"] / (2 << 30) - 1) < 0.01
