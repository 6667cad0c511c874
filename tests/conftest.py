import os
import sys

import pytest

# torch first: it carries its own HIP runtime, and libgdn.so must bind to that
# same runtime (loading the library first would map a second one).
import torch  # noqa: F401

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: full-size workload check")
