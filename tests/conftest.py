import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload checks")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library and a usable device; GPU tests fail loudly without them."""
    import torch
    from masked_attention_eagle_amd import ttt_attn
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    ttt_attn.load()  # raises if the shared library is missing
    return ttt_attn
