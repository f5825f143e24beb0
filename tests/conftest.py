import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device) and the built library")
    config.addinivalue_line("markers", "slow: full-size workload (long set-up)")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a HIP device exists; the CPU suite deselects them with -m "not gpu".
    pass
