import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library, on a machine with a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decoder_attention_g4attn_amd as g4
    g4.load()   # raises if the extension is missing: no fallback
    return g4
