import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # GPU tests need the device; skip them loudly when none is present so that the
    # CPU suite stays green on a machine without one, while "-m gpu" on an MI355X runs them.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# Error figures that passing GPU parity tests print (their "max-abs ..." lines) are
# collected and listed at the end of the run, so the errors are on record even when
# pytest captures a passing test's output.
_PARITY_LINES = []


def pytest_runtest_logreport(report):
    if report.when != "call" or not report.passed or "gpu" not in report.keywords:
        return
    name = report.nodeid.split("::")[-1]
    for line in report.capstdout.splitlines():
        if "max-abs" in line or "bit-identical" in line or "sum rule" in line:
            _PARITY_LINES.append(f"{name}: {line.strip()}")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if _PARITY_LINES:
        terminalreporter.section("errors against the oracle (passing GPU tests)")
        for line in _PARITY_LINES:
            terminalreporter.write_line(line)
