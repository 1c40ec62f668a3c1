import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # build only what is missing; a present library is used as it is
    from scatter_tile_gather_amd import build as stg_build

    if not os.path.exists(stg_build.LIB):
        stg_build.build()
    import oracle

    oracle.build(force=False)


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def stg():
    """The product binding over the in-tree HIP library."""
    import scatter_tile_gather_amd as stg

    stg.load_library()
    return stg
