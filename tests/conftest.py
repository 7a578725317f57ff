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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_libraries():
    """Builds the HIP library (hipcc cross-compiles without a GPU) and the
    oracle when nothing is built yet; a built library is used as it is."""
    from sparse_attention_indexer_row_amd import _lib
    import oracle

    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_indexer_row_amd import build as hip_build
        hip_build.build()
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    yield
