"""The streaming-read probe runs, reads what it is given and leaves its sink alone (the fold of a buffer of
equal bytes is zero, never the value that would trigger the store)."""
import pytest
import torch

from long_context_decode_attn_amd import ops


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes,wgs", [(1 << 26, 512), ((1 << 20) + 48, 64), (16, 1)])
def test_stream_read_runs_and_writes_nothing(nbytes, wgs):
    buf = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    ops.stream_read(buf, wgs, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 12345


@pytest.mark.gpu
def test_stream_read_rejects_odd_sizes():
    with pytest.raises(ValueError):
        ops.stream_read(torch.zeros(17, dtype=torch.uint8, device="cuda"), 4)
