import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of oracle time)")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture
def overrides():
    """Force launch choices for one test (tp_set_test_overrides); restored afterwards."""
    from tensor_transformer_layers_amd import binding as B

    def set_(spec):
        B.check(B.tp_set_test_overrides(spec))

    yield set_
    B.tp_set_test_overrides(None)
