import os
import sys

import pytest

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    import torch

    has_gpu = torch.cuda.is_available()
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords and not has_gpu:
            it.add_marker(skip)


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # name the case on the real stderr before any GPU work starts, so that a
    # run that ends abruptly still says which case it was in
    if "gpu" in request.node.keywords:
        sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
