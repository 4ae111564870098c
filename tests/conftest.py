import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# every library call in the tests waits for its work and reports a device
# error against the entry point that enqueued it (see the binding's _done)
os.environ.setdefault("KRON_DELTA_SYNC_CHECK", "1")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    oracle.build(force=False)
