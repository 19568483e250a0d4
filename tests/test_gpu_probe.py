"""The read probe the bench compares the decode with: runs on buffers of any 16-byte multiple size,
one to four at a time, and rejects what it cannot read."""

import pytest
import torch

import quantized_kv_cache_store_amd as kvq
import gpu_util as U

pytestmark = pytest.mark.gpu


def test_stream_read_sizes():
    U.need_gpu()
    bufs = [torch.zeros(n, dtype=torch.uint8, device=U.DEV) for n in (16, 1040, 1 << 20, 3 * 1024 + 48)]
    kvq.debug_stream_read(bufs)
    kvq.debug_stream_read(bufs[:1])
    kvq.debug_stream_read([bufs[2], bufs[0]])
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        kvq.debug_stream_read(bufs + bufs[:1])
    with pytest.raises(kvq.KvqError):
        kvq.debug_stream_read([torch.zeros(24, dtype=torch.uint8, device=U.DEV)])
