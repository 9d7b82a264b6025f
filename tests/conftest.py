import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU case")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The float parity cases of the session: both error measures per case."""
    mod = sys.modules.get("tests.gpu_util")
    rows = getattr(mod, "REPORT", None) if mod else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "float parity: max-norm and floored element-wise relative error")
    for name, kernel, n, err, fl in rows:
        tr.write_line(f"{name:60.60s} {kernel:14.14s} n={n:<10d} maxnorm={err:.3e} elementwise={fl:.3e}")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when the device is missing but -m gpu was asked for.
    pass
