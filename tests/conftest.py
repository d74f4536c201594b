import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: exhaustive CPU sweeps of minutes; run with NVFP4_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("NVFP4_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive sweep of several minutes; set NVFP4_SLOW=1 to run it")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    oracle.lib()
    return oracle
