import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Print the cut margins the end-to-end GPU comparisons recorded."""
    mod = sys.modules.get("gpu_util")
    log = getattr(mod, "MARGIN_LOG", None) if mod else None
    if log:
        terminalreporter.write_sep("-", "cut margins (relative distance of the nearest decision from its cut)")
        for line in log:
            terminalreporter.write_line(line)
