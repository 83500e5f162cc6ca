import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def hip():
    """The HIP library binding; GPU tests fail loudly if it is not built."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    from rwkv_linear_attention_wkv7_amd import binding
    binding.lib()
    return binding
