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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU sweep")


@pytest.fixture(scope="session", autouse=True)
def _sanitized_oracle():
    """Under the sanitizer run (see tests/sanitizers.py) every oracle call
    goes to the sanitized build of the oracle."""
    import sanitizers
    d = sanitizers.sanitized_dir()
    if d is None:
        yield
        return
    import oracle
    with oracle.using_library(os.path.join(d, "liboracle.so")):
        yield
