import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The GPU tests fail loudly (never skip) when no device is present, so a
    machine without a working GPU cannot pass as green."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU (run with -m 'not gpu' on CPU)")
    import paged_kv_attention_amd as fi
    fi.load()  # raises if the HIP library is missing
    return torch.device("cuda:0")
