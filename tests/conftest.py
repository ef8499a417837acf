"""Shared pytest set-up: the ``gpu`` marker and the oracle fixtures."""
from __future__ import annotations

import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))
if str(Path(__file__).resolve().parent) not in sys.path:
    sys.path.insert(0, str(Path(__file__).resolve().parent))


# facts the GPU parity tests report at the end of the run (e.g. near-tie rows
# per full-size workload), printed even under -q
REPORT: list[str] = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    if REPORT:
        terminalreporter.write_sep("-", "parity report")
        for line in REPORT:
            terminalreporter.write_line(line)


@pytest.fixture(scope="session")
def oracle():
    from oracle.binding import Oracle
    return Oracle()
