import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a machine without one they are skipped rather than failed.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per (workload, check) with the parity figures the GPU tests measured: worst and
    mean absolute errors, LSE error, ulps, exact-rounding fraction, mismatched and near-tie rows."""
    from tests.parity_util import RECORDS, format_record
    if not RECORDS:
        return
    terminalreporter.write_sep("-", "parity summary (GPU vs float64 oracle)")
    for r in RECORDS:
        terminalreporter.write_line(format_record(r))
