import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size parity cases (minutes of oracle time)")


def pytest_runtest_logstart(nodeid, location):
    # Name each case on the real stdout before it runs, so a run that dies
    # inside a GPU call still shows which case it was.
    sys.__stdout__.write(f"[start] {nodeid}\n")
    sys.__stdout__.flush()
