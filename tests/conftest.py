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
    oracle.build()
    return oracle


# Full-size workloads shared by the GPU test modules (generated once per
# session: the MX configuration alone is 671M bf16 values).
@pytest.fixture(scope="session")
def token_major():
    from group_scaling_fp8_amd import workloads as wl
    return wl.token_major_gradient()


@pytest.fixture(scope="session")
def c5():
    from group_scaling_fp8_amd import workloads as wl
    return wl.c5_mx()
