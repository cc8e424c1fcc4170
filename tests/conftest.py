import os
import sys

import pytest

try:
    # torch first: the HIP library then binds to torch's HIP runtime (one
    # runtime per process), whatever order the test modules load it in.
    import torch  # noqa: F401
except ImportError:
    pass

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case, takes tens of seconds")


def pytest_runtest_setup(item):
    # GPU tests name their case before they touch the device, so that a run
    # that ends abruptly still says which case was running.
    if "gpu" in item.keywords:
        print(f"\n[gpu-case] {item.nodeid}", flush=True)
