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


@pytest.fixture
def prefill_variant():
    """Forces a form of the 16-bit prefill kernels for one test (restored to
    the planner's choice afterwards)."""
    import attention_flash_sdpa_amd as sdpa

    yield sdpa.set_prefill_variant
    sdpa.set_prefill_variant(None)
