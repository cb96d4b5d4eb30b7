import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "big: full-size (84.6M-row) GPU case")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a GPU; say so instead of failing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    # the largest err / limit each parity test saw, per check (tests/helpers.py)
    helpers = sys.modules.get("helpers")
    if helpers is None or not getattr(helpers, "RATIOS", None):
        return
    tr = terminalreporter
    tr.section("largest err/limit per parity test")
    for test, d in sorted(helpers.RATIOS.items()):
        tr.write_line(f"{test}: " + ", ".join(f"{k} {v:.3g}" for k, v in sorted(d.items())))
