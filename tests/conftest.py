import os
import sys

import pytest

# torch before the library in every test process (the library binds to the
# HIP runtime already loaded; see communication_gemm_amd/_native.py)
import torch  # noqa: F401,E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle
