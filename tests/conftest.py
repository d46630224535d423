import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")
    config.addinivalue_line("markers", "slow: full-size configuration (needs a GPU)")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built on first use)."""
    import oracle

    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def bsa_gpu():
    """The HIP library through its Python binding; skips when no GPU."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_inverse_amd as bsa

    bsa.abi_version()  # loads libbsa.so or raises
    return bsa
