"""pkv_stream_read, the read-ceiling reference the bench times next to a step:
it must read the whole 16-byte units of the range, in every launch shape the
bench uses, and nothing past them. A thread writes the sink only when the xor
of the words it loaded is a fixed value; the buffer is zero except for that
value in one unit, so the sink is written exactly when that unit is read."""

import numpy as np
import pytest

import paged_kv_cache_108_amd as pkv
from helpers import need_gpu

pytestmark = pytest.mark.gpu
MAGIC = 0x9E3779B9


@pytest.fixture(autouse=True)
def _gpu_present():
    need_gpu()


def _sink_after(torch, n16, unit, nbytes, unroll, blocks):
    words = np.zeros(4 * n16 + 8, dtype=np.uint32)
    words[4 * unit + 2] = MAGIC
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    pkv.stream_read(src, sink, nbytes=nbytes, blocks=blocks, unroll=unroll)
    torch.cuda.synchronize()
    return int(sink.cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("unroll,blocks", [(4, 512), (8, 256), (16, 2048), (16, 8192), (4, 1), (16, 3)])
@pytest.mark.parametrize("n16", [1, 255, 4099, 1 << 20])
def test_units_of_the_range_are_read_and_no_others(unroll, blocks, n16):
    torch = need_gpu()
    for unit in sorted({0, n16 // 2, n16 - 1}):
        assert _sink_after(torch, n16, unit, 16 * n16 + 7, unroll, blocks) == MAGIC, unit
    assert _sink_after(torch, n16, n16, 16 * n16 + 15, unroll, blocks) == 0      # past the range


def test_bad_arguments_are_refused():
    torch = need_gpu()
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for kw in [dict(unroll=3), dict(blocks=0), dict(blocks=(1 << 20) + 1)]:
        with pytest.raises(pkv.PkvError):
            pkv.stream_read(src, sink, **kw)
    with pytest.raises(ValueError):
        pkv.stream_read(src, sink, nbytes=257)
