import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity figures the GPU tests reported (max |gpu - oracle| per case), also when
    output capture hid them."""
    gpu_util = sys.modules.get("gpu_util")
    lines = getattr(gpu_util, "REPORT", [])
    errs = [line for line in lines if "max|err|" in line]
    if errs:
        terminalreporter.section("parity: max |gpu - oracle|")
        for line in errs:
            terminalreporter.write_line(line)
