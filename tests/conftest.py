import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.load()
    return oracle


@pytest.fixture
def rng():
    return np.random.default_rng(12345)


def pytest_sessionfinish(session, exitstatus):
    out = os.environ.get("HC_MARGIN_OUT")
    if not out:
        return
    try:
        import gpu_util
    except Exception:      # the GPU helpers were never imported
        return
    if gpu_util.MARGINS:
        import json
        with open(out, "w") as fh:
            json.dump(gpu_util.MARGINS, fh, indent=0)
