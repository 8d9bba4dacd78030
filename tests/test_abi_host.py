"""The C-ABI library on the host: it loads, exports what the header declares, and rejects
bad arguments with the documented status codes before anything reaches the GPU."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_86_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


@pytest.fixture(scope="module")
def lib():
    return pa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(pa.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_is_gfx950_code():
    data = open(pa.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings(lib):
    for code in (PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, -5):
        assert pa.status_string(code).startswith("PA_")
    assert pa.status_string(17) == "unknown pa_status"


def store(lib, k=FAKE, T=4, NB=8, BS=16, Hkv=2, D=128):
    return lib.pa_kvcache_store(k, FAKE, FAKE, T, FAKE, FAKE, NB, BS, Hkv, D, None)


def test_store_argument_checks(lib):
    assert store(lib, T=-1) == PA_ERR_SHAPE
    assert store(lib, D=96) == PA_ERR_UNSUPPORTED
    assert store(lib, BS=24) == PA_ERR_UNSUPPORTED
    assert store(lib, BS=2048) == PA_ERR_UNSUPPORTED
    assert store(lib, NB=0) == PA_ERR_SHAPE
    assert store(lib, Hkv=0) == PA_ERR_SHAPE
    assert store(lib, k=None) == PA_ERR_NULL
    assert store(lib, k=None, T=0) == PA_OK  # empty batch: nothing to do, nothing launched


def decode(lib, B=4, Hq=4, Hkv=2, D=128, BS=16, NB=64, MBS=8, q=FAKE, ws=FAKE, ws_bytes=None,
           out_dtype=0):
    if ws_bytes is None:
        ws_bytes = pa.decode_workspace_bytes(max(B, 1), Hq, Hkv if Hkv > 0 else 1, D, BS, MBS)
    return lib.pa_paged_decode(q, FAKE, FAKE, FAKE, MBS, FAKE, B, Hq, Hkv, D, BS, NB, 0.0, FAKE,
                               out_dtype, ws, ws_bytes, None)


def test_decode_argument_checks(lib):
    assert decode(lib, Hq=6, Hkv=4) == PA_ERR_SHAPE
    assert decode(lib, D=256) == PA_ERR_UNSUPPORTED
    assert decode(lib, BS=12) == PA_ERR_UNSUPPORTED
    assert decode(lib, out_dtype=7) == PA_ERR_UNSUPPORTED
    assert decode(lib, B=-1) == PA_ERR_SHAPE
    assert decode(lib, MBS=0) == PA_ERR_SHAPE
    assert decode(lib, q=None) == PA_ERR_NULL
    assert decode(lib, ws=None) == PA_ERR_WORKSPACE
    assert decode(lib, ws_bytes=16) == PA_ERR_WORKSPACE
    assert decode(lib, B=0, q=None) == PA_OK
    assert decode(lib, MBS=4097, BS=16, ws_bytes=1 << 30) == PA_ERR_UNSUPPORTED  # > 65536 tokens


def _ws(units, parts, D=128):
    """Decode workspace layout: per partial (unit, split slot, head) a (max, sum) pair, then
    D-float unnormalised outputs; each region rounded up to 256 bytes."""
    r = lambda x: -(-x // 256) * 256  # noqa: E731
    return r(parts * 8) + r(parts * D * 4)


def test_decode_workspace_sizes():
    # Qwen3-0.6B-shaped decode: 64 x 8 head groups, 16 splits of 256 tokens, 2 heads per group
    assert pa.decode_workspace_bytes(64, 16, 8, 128, 256, 16) == _ws(64 * 8, 64 * 8 * 16 * 2)
    assert pa.decode_workspace_bytes(0, 16, 8, 128, 256, 16) == 0
    # 128 x 8 head groups x 8 slots reach 8192 workgroups: splits of 512 tokens for contexts
    # above 8 x 256 (8 partial slots per head group instead of 16); the size is the most any
    # smaller batch needs, here 127 sequences with short splits
    assert pa.decode_workspace_bytes(128, 16, 8, 128, 256, 16) == _ws(127 * 8, 127 * 8 * 16 * 2)
    # with blocks smaller than a split the block ids stay in LDS: short splits only
    assert pa.decode_workspace_bytes(128, 16, 8, 128, 16, 256) == _ws(128 * 8, 128 * 8 * 16 * 2)
    assert pa.decode_workspace_bytes(4, 6, 4, 128, 16, 8) == 0  # 6 % 4 != 0
    assert pa.decode_workspace_bytes(4, 8, 4, 128, 16, 4097) == 0  # context above 65536 tokens
    # more query heads per KV head than one workgroup serves: split into sub-groups
    assert pa.decode_workspace_bytes(2, 32, 2, 64, 16, 4) > pa.decode_workspace_bytes(2, 16, 2, 64, 16, 4)


@pytest.mark.parametrize("shape", [(16, 8, 128, 256, 16, False), (16, 8, 128, 256, 16, True),
                                   (16, 8, 64, 512, 16, False), (2, 1, 128, 256, 256, False),
                                   (2, 1, 128, 256, 256, True), (28, 4, 128, 16, 512, False)])
def test_decode_workspace_never_shrinks_with_the_batch(shape):
    """A workspace sized for a batch serves every smaller batch (long splits, which halve the
    partial slots, switch on at a threshold batch)."""
    Hq, Hkv, D, BS, MBS, fp8 = shape
    f = pa.decode_fp8_workspace_bytes if fp8 else pa.decode_workspace_bytes
    sizes = [f(b, Hq, Hkv, D, BS, MBS) for b in range(1, 400)]
    assert all(x > 0 for x in sizes)
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))


def prefill(lib, B=2, Tq=10, mq=5, q=FAKE, D=128, BS=16, Hq=4, Hkv=2):
    return lib.pa_paged_prefill(q, FAKE, FAKE, FAKE, B, Tq, mq, FAKE, FAKE, FAKE, 8, FAKE, Hq, Hkv,
                                D, BS, 64, 0.0, FAKE, 0, None)


def test_prefill_argument_checks(lib):
    assert prefill(lib, B=-1) == PA_ERR_SHAPE
    assert prefill(lib, mq=11) == PA_ERR_SHAPE
    assert prefill(lib, D=80) == PA_ERR_UNSUPPORTED
    assert prefill(lib, Hq=5) == PA_ERR_SHAPE
    assert prefill(lib, q=None) == PA_ERR_NULL
    assert prefill(lib, Tq=0, q=None) == PA_OK


def test_prefill_fp8_argument_checks(lib):
    def pf8(B=2, Tq=10, mq=5, q=FAKE, D=128, BS=16, Hq=4, Hkv=2, ks=0.5, vs=0.5):
        return lib.pa_paged_prefill_fp8(q, FAKE, B, Tq, mq, FAKE, FAKE, FAKE, 8, FAKE, Hq, Hkv, D,
                                        BS, 64, 0.0, ks, vs, FAKE, 0, None)
    assert pf8(B=-1) == PA_ERR_SHAPE
    assert pf8(mq=11) == PA_ERR_SHAPE
    assert pf8(D=80) == PA_ERR_UNSUPPORTED
    assert pf8(Hq=5) == PA_ERR_SHAPE
    assert pf8(ks=0.0) == PA_ERR_SHAPE
    assert pf8(vs=float("inf")) == PA_ERR_SHAPE
    assert pf8(q=None) == PA_ERR_NULL
    assert pf8(Tq=0, q=None) == PA_OK


def test_gather_argument_checks(lib):
    def gather(B=2, maxc=40, cache=FAKE, BS=16):
        return lib.pa_paged_gather(cache, FAKE, 4, FAKE, FAKE, B, maxc, 2, 64, BS, 16, FAKE, None)
    assert gather(B=-3) == PA_ERR_SHAPE
    assert gather(BS=3) == PA_ERR_UNSUPPORTED
    assert gather(cache=None) == PA_ERR_NULL
    assert gather(B=0, cache=None) == PA_OK


def test_stream_read_argument_checks(lib):
    def probe(src=FAKE, nbytes=4096, sink=FAKE):
        return lib.pa_stream_read(src, nbytes, sink, None)
    assert probe(nbytes=0, src=None) == PA_OK
    assert probe(src=None) == PA_ERR_NULL
    assert probe(sink=None) == PA_ERR_NULL
    assert probe(nbytes=4100) == PA_ERR_SHAPE
    assert probe(src=ctypes.c_void_p(0x1008)) == PA_ERR_SHAPE
    assert probe(sink=ctypes.c_void_p(0x1002)) == PA_ERR_SHAPE


def test_python_binding_rejects_cpu_tensors():
    import torch
    k = torch.zeros(2, 1, 64, dtype=torch.bfloat16)
    cache = torch.zeros(4, 16, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        pa.kvcache_store(k, k, torch.zeros(2, dtype=torch.int32), cache, cache)


def test_store_fp8_argument_checks(lib):
    def store8(T=4, D=128, BS=16, ks=1.0, vs=1.0, k=FAKE):
        return lib.pa_kvcache_store_fp8(k, FAKE, FAKE, T, FAKE, FAKE, 8, BS, 2, D, ks, vs, None)
    assert store8(T=-1) == PA_ERR_SHAPE
    assert store8(D=96) == PA_ERR_UNSUPPORTED
    assert store8(BS=5) == PA_ERR_UNSUPPORTED
    assert store8(ks=0.0) == PA_ERR_SHAPE
    assert store8(vs=-2.0) == PA_ERR_SHAPE
    assert store8(ks=float("inf")) == PA_ERR_SHAPE
    assert store8(vs=float("nan")) == PA_ERR_SHAPE
    assert store8(k=None) == PA_ERR_NULL
    assert store8(T=0, k=None) == PA_OK


def test_decode_fp8_argument_checks(lib):
    def dec8(B=4, Hq=4, Hkv=2, D=128, ks=0.5, vs=0.5, q=FAKE, ws_bytes=None, MBS=8):
        if ws_bytes is None:
            ws_bytes = pa.decode_fp8_workspace_bytes(max(B, 1), Hq, Hkv, D, 16, MBS)
        return lib.pa_paged_decode_fp8(q, FAKE, FAKE, FAKE, MBS, FAKE, B, Hq, Hkv, D, 16, 64, 0.0,
                                       ks, vs, FAKE, 0, FAKE, ws_bytes, None)
    assert dec8(Hq=6, Hkv=4) == PA_ERR_SHAPE
    assert dec8(D=32) == PA_ERR_UNSUPPORTED
    assert dec8(ks=0.0) == PA_ERR_SHAPE
    assert dec8(vs=float("inf")) == PA_ERR_SHAPE
    assert dec8(q=None) == PA_ERR_NULL
    assert dec8(ws_bytes=8) == PA_ERR_WORKSPACE
    assert dec8(B=0, q=None) == PA_OK
    assert dec8(MBS=4097, ws_bytes=1 << 30) == PA_ERR_UNSUPPORTED


def test_decode_fp8_workspace_sizes():
    # Same short split length as bf16 (256 tokens at head_dim 128), but FP8 pools take long
    # splits from grids of 1024 workgroups (bf16: 8192): 64 sequences x 8 KV heads with 16
    # short slots get 8 long ones, twice as long, where bf16 keeps 16.
    assert pa.decode_fp8_workspace_bytes(64, 16, 8, 128, 256, 16) == _ws(64 * 8, 64 * 8 * 8 * 2)
    assert pa.decode_workspace_bytes(64, 16, 8, 128, 256, 16) == _ws(64 * 8, 64 * 8 * 16 * 2)
    # 8 heads per KV head run the MFMA kernel on both pools (no long splits there)
    assert pa.decode_fp8_workspace_bytes(64, 64, 8, 128, 16, 64) == \
        pa.decode_workspace_bytes(64, 64, 8, 128, 16, 64)
    # a group of 5 runs the MFMA kernel (bf16 and FP8): one workgroup of 5 heads; a group of 2
    # on FP8 runs the VALU kernel, and 20 heads per KV head the MFMA kernel as two of 10
    assert pa.decode_workspace_bytes(1, 5, 1, 128, 256, 16) == _ws(1, 16 * 5)
    assert pa.decode_fp8_workspace_bytes(1, 5, 1, 128, 256, 16) == _ws(1, 16 * 5)
    assert pa.decode_fp8_workspace_bytes(1, 2, 1, 128, 256, 16) == _ws(1, 16 * 2)
    assert pa.decode_fp8_workspace_bytes(1, 20, 1, 128, 256, 16) == _ws(2, 16 * 20)
    assert pa.decode_fp8_workspace_bytes(4, 6, 4, 128, 16, 8) == 0


def test_decode_append_argument_checks(lib):
    def app(B=4, Hq=4, Hkv=2, D=128, k_new=FAKE, slots=FAKE, ws_bytes=None, fp8=False):
        if ws_bytes is None:
            ws_bytes = pa.decode_workspace_bytes(max(B, 1), Hq, Hkv, D, 16, 8)
        if fp8:
            return lib.pa_paged_decode_append_fp8(FAKE, k_new, FAKE, slots, FAKE, FAKE, FAKE, 8,
                                                  FAKE, B, Hq, Hkv, D, 16, 64, 0.0, 1.0, 0.0,
                                                  FAKE, 0, FAKE, ws_bytes, None)
        return lib.pa_paged_decode_append(FAKE, k_new, FAKE, slots, FAKE, FAKE, FAKE, 8, FAKE, B,
                                          Hq, Hkv, D, 16, 64, 0.0, FAKE, 0, FAKE, ws_bytes, None)
    assert app(k_new=None) == PA_ERR_NULL
    assert app(slots=None) == PA_ERR_NULL
    assert app(B=0, k_new=None) == PA_OK
    assert app(D=80) == PA_ERR_UNSUPPORTED
    assert app(ws_bytes=4) == PA_ERR_WORKSPACE
    assert app(fp8=True) == PA_ERR_SHAPE  # v_scale 0


def test_decode_append_noalloc_argument_checks(lib):
    """Argument errors come back before any device call; a size whose workspace exceeds the
    fixed scratch array is refused with PA_ERR_SCRATCH."""
    def app(B=4, Hq=4, Hkv=2, D=128, BS=16, MBS=8, k_new=FAKE, q=FAKE):
        return lib.pa_paged_decode_append_noalloc(q, k_new, FAKE, FAKE, FAKE, FAKE, FAKE, MBS,
                                                  FAKE, B, Hq, Hkv, D, BS, 64, 0.0, FAKE, 0, None)
    assert app(k_new=None) == PA_ERR_NULL
    assert app(q=None) == PA_ERR_NULL
    assert app(B=0, k_new=None) == PA_OK
    assert app(D=80) == PA_ERR_UNSUPPORTED
    assert app(Hq=6, Hkv=4) == PA_ERR_SHAPE
    # 7B-shaped decode at 256 sequences with 65,536-token tables needs ~119 MB of partials
    # (the most any batch up to 256 needs): above the 64 MiB scratch
    assert pa.decode_workspace_bytes(256, 28, 4, 128, 16, 4096) > pa.DECODE_SCRATCH_BYTES
    assert app(B=256, Hq=28, Hkv=4, BS=16, MBS=4096) == pa.PA_ERR_SCRATCH
    assert pa.status_string(pa.PA_ERR_SCRATCH).startswith("PA_ERR_SCRATCH")
    # the Qwen3-0.6B-shaped, 7B-shaped (8,192-token tables) and 512-sequence decodes fit
    for args in ((64, 16, 8, 128, 256, 16), (256, 28, 4, 128, 16, 512), (512, 16, 8, 128, 256, 16)):
        assert 0 < pa.decode_workspace_bytes(*args) <= pa.DECODE_SCRATCH_BYTES


def test_decode_graph_argument_checks(lib):
    h = ctypes.c_void_p()

    def create(max_batch=8, Hq=4, Hkv=2, D=128, out_dtype=0, kc=FAKE, handle=True):
        return lib.pa_decode_graph_create(max_batch, Hq, Hkv, D, 16, 64, 8, 0, 0.0, 1.0, 1.0, kc,
                                          FAKE, out_dtype, ctypes.byref(h) if handle else None)
    assert create(handle=False) == PA_ERR_NULL
    assert create(max_batch=0) == PA_ERR_SHAPE
    assert create(max_batch=70000) == PA_ERR_SHAPE
    assert create(kc=None) == PA_ERR_NULL
    assert create(out_dtype=3) == PA_ERR_UNSUPPORTED
    assert create(Hq=6, Hkv=4) == PA_ERR_SHAPE  # no workspace size for these heads
    assert h.value is None
    assert lib.pa_decode_graph_run(None, 1, None, None, None, None, None, 1, None, None,
                                   None) == PA_ERR_NULL
    assert lib.pa_decode_graph_bucket(None, 3) == 0
    assert lib.pa_decode_graph_destroy(None) == PA_OK
