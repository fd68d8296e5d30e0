import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X); runs through the C ABI")
    config.addinivalue_line("markers", "slow: large synthetic workloads")


_CACHE = {}


@pytest.fixture(scope="session")
def workload():
    """Generate (and cache) a named synthetic workload."""
    from entropy_decoding_df11_amd import workloads

    def get(name):
        if name not in _CACHE:
            _CACHE[name] = workloads.make(name)
        return _CACHE[name]

    return get
