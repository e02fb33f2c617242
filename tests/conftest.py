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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) device and the built HIP library")


@pytest.fixture(autouse=True)
def _name_gpu_case(request):
    """Print (and flush) the id of every GPU test before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield


def pytest_terminal_summary(terminalreporter):
    """Print the parity lines the GPU tests recorded (worst rows against the oracle)."""
    util = sys.modules.get("gpu_util")
    if util is not None and getattr(util, "REPORT", None):
        terminalreporter.write_sep("-", "parity against the float64 oracle")
        for line in util.REPORT:
            terminalreporter.write_line(line)
