"""The streaming-read reference (kvq_stream_read): it reads one to four buffers of any
16-byte multiple without touching the sink (the sink is written only if a workgroup's
folded data equals a fixed constant, which the data below cannot give)."""
import pytest
import torch

from bit_kv_cache_pack_amd import kvq as K

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sizes", [(4096,), (16, 48, 4096 + 16), (1 << 20, 3 << 16, 160, 1 << 22),
                                   ((1 << 16) + 16,), (42303488 // 2,)])
def test_stream_read_leaves_sink(sizes):
    from gpu_common import DEV
    print(f"[stream_read] sizes={sizes}", flush=True)
    bufs = [torch.zeros(n, dtype=torch.uint8, device=DEV) for n in sizes]
    sink = torch.full((64,), 7, dtype=torch.int32, device=DEV)
    K.kvq_stream_read(bufs, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 7)
