import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a host without one they are skipped, not
    # failed, so that `-m "not gpu"` and plain runs both work here.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _checked_build_finds_nothing(request):
    """With DSA_LIBRARY=debug (every call through the checked build), each
    GPU test must leave the checked build's fault word clear: no metadata
    outside its bounds, no output element left unwritten, no invalid
    selection row.  Tests that plant bad metadata read and clear the word
    themselves."""
    if os.environ.get("DSA_LIBRARY") != "debug" or "gpu" not in request.keywords:
        yield
        return
    import sparse_attention_topk_amd as dsa
    dsa.debug_faults(clear=True)
    yield
    faults = dsa.debug_faults(clear=True)
    assert faults == 0, "checked build raised fault bits 0x%x" % faults
