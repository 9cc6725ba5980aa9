import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def fd():
    """The HIP library binding, on a GPU. Fails loudly if the library is missing."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_decoding_amd as fdmod
    fdmod.load_library()
    return fdmod
