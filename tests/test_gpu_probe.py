"""Measurement aids, not part of the attention path: the streaming-read probe runs on sizes
that do and do not fill its grid and rejects misaligned sizes before launching; the decode
timing request brackets the next decode call's main kernel only."""
import pytest
import torch

import paged_kv_cache_86_amd as pa
from gpu_util import DecodeOnDevice, device, say
from workloads import decode_case

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


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (28, 4)], ids=["valu", "mfma"])
def test_decode_time_next_launch_brackets_the_split_kernel(Hq, Hkv):
    """The two events land around the next decode call's split kernel: a positive interval no
    longer than the whole call (store of the request, the kernel, the merge); the request is
    used up, so a following call leaves the events as they were."""
    dev = device()
    c = decode_case(77, [300, 1200, 17, 4000], Hq, Hkv, 128, 16, nb_factor=1.2)
    d = DecodeOnDevice(c, dev)
    say(f"[timing] {Hq}/{Hkv} heads")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    ev[2].record()
    pa.decode_time_next_launch(ev[0], ev[1])
    d.decode()
    ev[3].record()
    torch.cuda.synchronize()
    inner, whole = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    say(f"[timing] split kernel {inner * 1e3:.1f} us of {whole * 1e3:.1f} us")
    assert 0 < inner <= whole
    d.decode()
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == inner
