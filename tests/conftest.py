import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload")


def pytest_collection_modifyitems(config, items):
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


# Parity figures that tests record (workload, tensor, max-abs-rel, tolerance)
# are printed in the terminal summary, so that a quiet (-q) run shows them.
def pytest_terminal_summary(terminalreporter, exitstatus, config):
    from parity_log import PARITY
    if not PARITY:
        return
    terminalreporter.section("parity (max-abs-rel over the whole tensor)")
    for name, tensor, err, tol in PARITY:
        terminalreporter.write_line(f"{name:<34} {tensor:<14} {err:.3e}  (tolerance {tol:g})")
