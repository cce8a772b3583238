import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large oracle work (full-size sampled parity)")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name every GPU case (test id, parameters) on stderr before it runs, so a
    run that dies inside a kernel still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield


@pytest.fixture(scope="session")
def cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X; none is available")
    from w8a8_int8_linear_amd import _lib

    _lib.load()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")
