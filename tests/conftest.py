import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")
    config.addinivalue_line("markers", "slow: full-size workload checks")


def pytest_sessionstart(session):
    """Build the native libraries only when nothing is built yet."""
    import os
    lib = os.path.join(ROOT, "pooling_tbe_forward_amd", "libtbe.so")
    if not os.path.exists(lib):
        from pooling_tbe_forward_amd import build
        build.build()
    import oracle
    oracle.build()
