"""The streaming-read probe (a measurement aid, not part of the attention path) runs on sizes
that do and do not fill its grid, and rejects misaligned sizes before launching."""
import pytest
import torch

import paged_kv_cache_86_amd as pa
from gpu_util import device, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1 << 20, (64 << 20) + 48])
def test_stream_read_sizes(nbytes):
    dev = device()
    say(f"[probe] {nbytes} bytes")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    pa.stream_read(src, sink)
    torch.cuda.synchronize()


def test_stream_read_rejects_partial_words():
    dev = device()
    src = torch.ones(5, dtype=torch.float32, device=dev)  # 20 bytes
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(pa.PagedAttnError):
        pa.stream_read(src, sink)
