import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check, skipped unless WT_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("WT_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow CPU check; set WT_SLOW=1 to run")
    for it in items:
        if "slow" in it.keywords and "gpu" not in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    if os.environ.get("WT_ORACLE_LIB"):
        return oracle
    src = os.path.join(oracle.HERE, "oracle.c")
    stale = not os.path.exists(oracle.LIB_PATH) or os.path.getmtime(oracle.LIB_PATH) < os.path.getmtime(src)
    if stale:
        oracle.build()
    return oracle
