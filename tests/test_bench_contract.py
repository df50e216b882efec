"""bench.py: its command-line contract and the counter summaries it quotes.

CPU only.  The benchmark reports HBM traffic from the committed rocprofv3
summaries under profiles/ only while they were taken from the HB kernel's
current sources; these tests hold that link, and check that a request for more
than one GPU is refused with a message (the R ranks are simulated on one GPU).
"""
import importlib.util
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)
    assert not res.stdout.strip().startswith("{"), "no JSON line for an unsupported run"


def test_counter_summaries_match_the_hb_sources(bench):
    """The committed counter readings belong to the HB kernel as it is now
    compiled; after a change to hb_twoshot.hip, ar_device.hpp or the flags,
    retake them (and until then the bench reports traffic as null)."""
    b8 = bench._counter_traffic()
    assert b8 is not None, "profiles/hb_twoshot_bf16_r8_128MiB_counters.txt is stale"
    # 8 ranks x 128 MiB read once and written once: 2 GiB of algorithmic bytes
    assert abs(b8 / (2 << 30) - 1.0) < 0.01
    for key, ranks in (("hbm_bytes_per_launch_r16", 16), ("hbm_bytes_per_launch_r32", 32)):
        got = bench._counter_traffic(bench.C5B_COUNTERS, key)
        assert got is not None, f"profiles/{bench.C5B_COUNTERS} is stale"
        assert abs(got / (2 * ranks * bench.C5B_BYTES) - 1.0) < 0.01


def test_stale_summary_reads_as_null(bench, tmp_path, monkeypatch):
    """A summary whose digest does not match yields None, never a number."""
    src = ROOT / "profiles" / "hb_twoshot_bf16_r8_128MiB_counters.txt"
    text = src.read_text().replace("source_sha256: ", "source_sha256: 00")
    fake_root = tmp_path / "repo"
    (fake_root / "profiles").mkdir(parents=True)
    (fake_root / "profiles" / src.name).write_text(text)
    monkeypatch.setattr(bench, "__file__", str(fake_root / "bench.py"))
    monkeypatch.setattr(bench, "_sources_digest", lambda: "not-the-digest")
    assert bench._counter_traffic() is None
