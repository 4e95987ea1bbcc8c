import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size configurations)")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as o
    o.build()
    return o.default()


@pytest.fixture(params=[1, 0], ids=["unit", "chunked"])
def topk_kernel(request):
    """Both TOPK forms: one launch with the distances in LDS and a histogram exchange (the default where the
    grid fits the device) and the chunked histogram + compaction passes."""
    from long_context_decode_attn_amd import ops
    old = ops.get_tuning("topk_kernel")
    ops.set_tuning("topk_kernel", request.param)
    yield request.param
    ops.set_tuning("topk_kernel", old)
