import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library and a visible device, or a loud failure where a device is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from block_diffusion_drafter_target_amd import binding
    return binding.load()
