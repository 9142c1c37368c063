import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()
    # the HIP library too, if nothing is built yet (a fresh checkout: built
    # libraries are not in version control); an existing build is used as is
    from attention_non_causal_amd import _lib
    from attention_non_causal_amd import build as libbuild
    if not os.path.exists(_lib.LIB_PATH) and libbuild.hipcc():
        libbuild.build()
    if not os.path.exists(_lib.DEBUG_LIB_PATH) and libbuild.hipcc():
        libbuild.build(debug_barriers=True)
    if not os.path.exists(libbuild.PROBE_LIB_PATH) and libbuild.hipcc():
        libbuild.build_probe()
    yield
