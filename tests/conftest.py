import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded through its Python binding (GPU tests only)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from newton_schulz_matrix_muon_amd import muon

    # every step and NS call of the GPU tests waits for its stream and
    # raises if a persistent launch stopped early
    muon.check_default = True
    return muon
