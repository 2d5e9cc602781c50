import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them with a clear reason
    # rather than failing when the CPU suite is run without -m selection.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    # the full-size parity checks' error summaries (max error against the
    # tolerance bound), when GPU tests ran in this session
    g = sys.modules.get("tests._gpu")
    lines = getattr(g, "SUMMARY", None)
    if lines:
        terminalreporter.write_sep("-", "parity error summaries")
        for line in lines:
            terminalreporter.write_line(line)
