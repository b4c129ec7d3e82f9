import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; fails, not skips, without one")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The native library on cuda:0. A GPU test without a device fails."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test requires a ROCm device (none visible)")
    from qlora_adapter_amd import nf4lora
    nf4lora.load()
    return nf4lora
