import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    # Name the case before it runs, so a run that dies mid-test still says which.
    if "gpu" in item.keywords:
        print(f"\n[gpu-case] {item.nodeid}", flush=True)
