import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    from oracle import oracle as O
    O.lib()
    return O


def to_bits_u16(t):
    """torch bf16 tensor -> numpy uint16 bit patterns."""
    from sparse_mixture_experts_08_amd.workloads import to_numpy
    return to_numpy(t)
