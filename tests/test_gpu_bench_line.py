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
    line = _run("--only", "sweep", "--steps", "2", "--warmup", "1", "--no-cpu")
    _contract(line, 2, 1)
    rows = line["ll_sweep"]
    assert [r["bytes_per_rank"] for r in rows] == [2 << k for k in range(10, 20)]
    assert all(r["ll_parity"] and r["hb_parity"] for r in rows)
    # the graph's own first replay (outputs zeroed after capture) is exact too
    assert all(r["ll_parity_graph"] and r["hb_parity_graph"] for r in rows)
    dec = line["decode_64x8192"]
    assert dec["ll_parity_graph"] and dec["hb_parity_graph"]
    assert line["value"] == pytest.approx(sum(r["ll_us"] for r in rows) / len(rows), abs=2e-3)
    # the floor is a one-workgroup call: below the slowest LL call on any machine
    assert 0 < line["graph_floor_us"] < max(r["ll_us"] for r in rows)
    assert line["ll_mean_above_floor_us"] == pytest.approx(
        line["value"] - line["graph_floor_us"], abs=2e-3)
    assert line["ms_per_step"] == pytest.approx(sum(r["ll_us"] for r in rows) * 10 / 1000,
                                                abs=1e-3)
    # every row names the launch it timed: LL with 8-byte packets at the
    # built-in shape, HB with one kernel
    for r in rows:
        assert r["ll_launch"]["packetBytes"] == 8 and r["ll_launch"]["grid"] % 8 == 0
        assert r["hb_launch"]["kernels"] == 1 and r["hb_launch"]["grid"] % 8 == 0
        assert r["ll_us_median"] > 0 and r["hb_us_median"] > 0
    assert line["value_median_passes"] == pytest.approx(
        sum(r["ll_us_median"] for r in rows) / len(rows), abs=2e-3)
    assert line["config"]["tuned"] is False
    c1 = line["c1"]
    assert c1["ll_parity"] and c1["hb_parity"] and c1["elems_per_rank"] == 1024


def test_prefill_roofline():
    line = _run("--only", "prefill", "--steps", "3", "--warmup", "1", "--no-cpu")
    _contract(line, 3, 1)
    assert line["hb_prefill"]["parity"] is True
    # the graph-replayed figure of the same in-place calls, beside the back-to-back one
    assert 0.5 < line["hb_prefill"]["us_graph"] / line["hb_prefill"]["us_per_launch"] < 2
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["bytes_per_launch"] == 2 << 30
    assert roof["achieved"] == pytest.approx(
        roof["bytes_per_launch"] / (roof["us_per_launch"] * 1e-6) / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    # traffic is the committed counter reading (checked against the sources on the CPU)
    assert roof["traffic"] is None or abs(roof["traffic"] / (2 << 30) - 1) < 0.01


def test_c5_rows():
    """C5 at R = 16 and 32: both HB chunk layouts (chunk = N/R as configured,
    and interleaved tiles), LL at the fp16 size; every row bit-exact against
    the oracle and equal to the exact integer sums."""
    line = _run("--only", "c5", "--steps", "2", "--warmup", "1", "--no-cpu")
    _contract(line, 2, 1)
    rows = line["c5"]
    assert len(rows) == 2 * 3 + 2 * 2
    assert all(r["parity"] and r["exact_integer_sums"] for r in rows)
    assert {r["chunk_layout"] for r in rows if r["proto"] == "hb"} == {"chunk N/R",
                                                                          "interleaved tiles"}
    for r in rows:
        assert r["gbps"] == pytest.approx(
            2 * r["R"] * r["bytes_per_rank"] / (r["us"] * 1e-6) / 1e9, rel=2e-3)
    # C5b is also timed per call with the last-level cache flushed first
    for r in rows:
        if r["config"] == "C5b":
            assert 0 < r["us_cold_median"] and 0 < r["us_cold_mean"]
        else:
            assert "us_cold_mean" not in r
