import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def built_lib():
    """Path of libgqa.so; compiled here only when nothing is built yet."""
    from grouped_query_attention_02_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from grouped_query_attention_02_amd import build
        build.build()
    return _lib.LIB_PATH
