import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    """Worst GPU-vs-oracle output margins of this run, per workload or shape
    (bar: max-abs 2e-2, mean-abs 2e-3)."""
    try:
        from _parity import MARGINS
    except ImportError:
        return
    if not MARGINS:
        return
    tr = terminalreporter
    tr.write_sep("-", "GPU vs oracle output margins (worst per label; bar max-abs 2e-2, mean-abs 2e-3)")
    for label in sorted(MARGINS):
        mx, mean, n = MARGINS[label]
        tr.write_line(f"{label[:72]:72s} max-abs {mx:.3e}  mean-abs {mean:.3e}  ({n} comparisons)")
