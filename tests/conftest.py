import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built libdecodegemv")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr before it runs, so a run that ends the
    process still shows which case was in flight."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield


@pytest.fixture(scope="session")
def dg():
    """The Python binding of libdecodegemv, on a GPU machine."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import memory_bound_decode_gemv_amd as m
    m.raw()   # raises if the library is not built
    return m


@pytest.fixture(scope="session")
def dev():
    import torch
    return torch.device("cuda:0")
