import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger oracle cases")


def pytest_collection_modifyitems(config, items):
    # every test in a test_gpu_* module needs the GPU
    for it in items:
        if os.path.basename(str(it.fspath)).startswith("test_gpu_") and "gpu" not in it.keywords:
            it.add_marker(pytest.mark.gpu)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    # the layer tests' parity statistics (outputs beyond the tolerance, act
    # code flips), so that a quiet run still shows them
    try:
        from tests.gpu_helpers import PARITY_RECORD
    except Exception:
        return
    if PARITY_RECORD:
        terminalreporter.write_sep("-", "parity record")
        for rec in PARITY_RECORD:
            terminalreporter.write_line(" ".join(f"{k}={v}" for k, v in rec.items()))
