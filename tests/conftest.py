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


def pytest_sessionstart(session):
    """Build the oracle, if it is missing or stale, before any test runs:
    at this point no test has touched the GPU, so starting a compiler is
    safe.  The oracle itself never compiles on load."""
    import oracle
    if oracle.is_stale():
        oracle.build(force=True)


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle


def pytest_runtest_setup(item):
    """GPU tests fail (never skip) on a machine without a GPU, so a silent
    skip can never pass for a parity result."""
    if item.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("test marked gpu but no GPU is visible")
        print(f"\n[gpu case] {item.nodeid}", flush=True)


def pytest_sessionfinish(session, exitstatus):
    """With QL_TOLERANCE_REPORT=<path>, write the float-check reports (the
    fraction of entries meeting the stated bound alone, the largest
    err / stated bound, per check) to that file."""
    path = os.environ.get("QL_TOLERANCE_REPORT")
    if not path:
        return
    import json
    from tolerance import REPORTS
    Path(path).parent.mkdir(parents=True, exist_ok=True)
    Path(path).write_text(json.dumps(REPORTS, indent=1))
