import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def cca_lib():
    """The built libcca.so (built in-tree first when it is missing)."""
    from sparse_long_context_cca_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_long_context_cca_amd import build
        build.build(verbose=False)
    return _lib.load()
