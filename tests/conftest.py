import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


@pytest.fixture(autouse=True)
def _wkv_waits_never_ran_out(request):
    """Around every GPU test: the bounded in-workgroup waits of the WKV kernels never ran out
    (the library counts each one that did on the device)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import torch

    if not torch.cuda.is_available():
        yield
        return
    from linear_recurrence_chunked_amd import lrc

    lrc.wait_timeouts(reset=True)
    yield
    assert lrc.wait_timeouts() == 0, "a bounded wait inside a WKV kernel ran out"
