import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    import report
    if report.GAP_STATS or report.LINES:
        terminalreporter.write_sep("-", "parity figures")
        for line in report.LINES:
            terminalreporter.write_line(str(line))
        if report.GAP_STATS:
            terminalreporter.write_line(
                "Top-k sets vs the oracle, by the k-th/(k+1)-th gap against tau_r "
                "[rows, rows equal to the exact sort prefix]: " + str(report.GAP_STATS))
