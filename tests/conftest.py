import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """How often the weight-gradient max checks needed the rounding-flip allowance."""
    mod = sys.modules.get("tests.gpu_util")
    line = mod.allowance_summary() if mod is not None else None
    if line:
        terminalreporter.write_line(line)
