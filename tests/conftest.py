import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size workload, minutes of host work")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0; skips only when there is no GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_mqa_logits_indexer_amd as lib  # raises if the .so is missing
    lib.load_library()
    return lib
