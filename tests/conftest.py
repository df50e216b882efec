"""Shared pytest set-up: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything else
runs on the CPU.
"""
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
for p in (ROOT, ROOT / "tests"):
    if str(p) not in sys.path:
        sys.path.insert(0, str(p))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.load()
