import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case, minutes of CPU work")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as o
    o.build()
    o.set_mutation(0)
    return o


@pytest.fixture(scope="session")
def q4():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_matmul_q4_amd as m
    m.lib()  # raises if the library is missing
    return m
