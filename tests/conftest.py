"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything
else runs on the CPU (oracle pins, host-side argument validation, symbol
exports of the C-ABI library).
"""
import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


def read_golden(name):
    """Yield the whitespace-split, non-comment lines of a golden fixture."""
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        yield line.split()


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_runtest_setup(item):
    """GPU tests fail (never skip) on a machine without a GPU, so a silent
    skip can never pass for a parity result."""
    if item.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("test marked gpu but no GPU is visible")
        print(f"\n[gpu case] {item.nodeid}", flush=True)
