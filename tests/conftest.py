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
    # GPU tests cannot run without a device: skip them (with the reason) rather than fail.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    # achieved errors of the float parity comparisons (tests/helpers.py report()), one line each
    try:
        from tests.helpers import RESULTS
    except Exception:  # pragma: no cover
        return
    if not RESULTS:
        return
    tr = terminalreporter
    tr.section("achieved parity errors (max|err|/max|ref|; of_bar = share of the element-wise bar used)")
    for test, what, vals in RESULTS:
        tr.write_line(f"{test} | {what} | " + ", ".join(f"{k}={v:.3e}" for k, v in vals.items()))
