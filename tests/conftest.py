import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library on cuda:0; fails loudly when either is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    import exact_attention_118_amd as fa

    fa.load_library()
    return fa
