import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes of CPU oracle time)")


def read_table(name):
    """Rows of a whitespace table under tests/golden/, skipping '#' comments and the header."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
    return lines


@pytest.fixture(scope="session")
def golden():
    return read_table


@pytest.fixture(scope="session")
def full_bank():
    """The 896-expert bank of the layer workloads (15.7 GB of HBM), shared by the GPU tests."""
    import torch

    import mxfp4_moe_expert_amd as k3g
    import synth
    from tests.helpers import make_bank

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    print("generating the 896-expert bank", flush=True)
    src, bankt, bank = make_bank(k3g, synth.SEED_BASE + 1, 896, 3584, 3072)
    yield src, bankt, bank
    del bankt
    torch.cuda.empty_cache()
