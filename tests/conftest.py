import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def q4lib():
    """The built libq4gemv.so (compiled first only if it was never built)."""
    import bit_block_quantized_dequant_amd as q4
    if not os.path.exists(q4.LIB_PATH):
        from bit_block_quantized_dequant_amd import build
        build.build()
    return q4.lib()


@pytest.fixture(scope="module")
def dev():
    """cuda:0, for the GPU tests; fails loudly if the HIP library is missing."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_block_quantized_dequant_amd as q4
    q4.lib()
    return torch.device("cuda:0")
