"""Mixed prefill + decode in one call: chunks and one-token decode rows under one cu_seqlens_q,
against the oracle treating every row as a chunk row; the decode rows on a second stream give
bit-identical results; the degenerate mixes equal the single-kind calls."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_86_amd as pa
from gpu_util import as_f64, bf16, bits, device, i32, say
from workloads import mixed_case

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def run_mixed(c, n_chunks, dev, out_dtype=torch.float32, decode_stream=None, pools=None):
    kc, vc = pools if pools is not None else (bf16(c.k_cache, dev), bf16(c.v_cache, dev))
    T = c.total_q
    out = torch.empty((T, c.num_q_heads, c.head_dim), dtype=out_dtype, device=dev)
    prefill_tokens = int(c.cu_seqlens_q[n_chunks])
    mq = int(c.q_lens[:n_chunks].max()) if n_chunks else 0
    pa.paged_attention_mixed(bf16(c.q, dev), bf16(c.k_new, dev), bf16(c.v_new, dev),
                             i32(c.slot_mapping, dev), i32(c.cu_seqlens_q[:n_chunks + 1], dev),
                             i32(c.block_tables, dev), i32(c.context_lens, dev), out, k_cache=kc,
                             v_cache=vc, num_prefill_seqs=n_chunks, prefill_tokens=prefill_tokens,
                             max_prefill_q_len=mq, scale=c.scale, decode_stream=decode_stream)
    return out, kc, vc


def oracle_mixed(c):
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_prefill(c.q, c.k_new, c.v_new, c.cu_seqlens_q, kc, vc, c.block_tables,
                               c.context_lens, np.float32(c.scale))
    return ref, kc, vc


CASES = [
    # (D, BS, Hq, Hkv, chunk prefixes, chunk lengths, decode contexts)
    (128, 16, 8, 2, [0, 37, 300], [70, 1, 129], [1, 2, 17, 256, 700]),
    (64, 64, 4, 4, [130], [33], [65, 1000, 3, 64]),
    (128, 256, 16, 8, [512, 0], [200, 257], [4096, 300, 1]),
    (128, 16, 12, 2, [], [], [20, 600]),          # decode rows only
    (64, 16, 4, 1, [10, 90], [64, 5], []),        # chunks only
]


@pytest.mark.parametrize("case", CASES, ids=[f"D{c[0]}_bs{c[1]}_{len(c[4])}c{len(c[6])}d" for c in CASES])
def test_mixed_matches_oracle(case):
    dev = device()
    D, BS, Hq, Hkv, P, n, dctx = case
    c = mixed_case(600 + D + BS, P, n, dctx, Hq, Hkv, D, BS, num_blocks=None)
    say(f"[mixed] D={D} BS={BS} chunks={list(zip(P, n))} decodes={dctx}")
    ref, okc, ovc = oracle_mixed(c)
    for out_dtype in (torch.float32, torch.bfloat16):
        out, kc, vc = run_mixed(c, len(P), dev, out_dtype)
        torch.cuda.synchronize()
        err = np.abs(as_f64(out) - ref).max()
        say(f"[mixed]   {out_dtype}: max|err| {err:.3e}")
        assert err <= ATOL
        assert np.array_equal(bits(kc), okc) and np.array_equal(bits(vc), ovc)


def test_mixed_second_stream_equals_separate_calls():
    """With a second stream, every row is stored first, then the decode rows run as a plain
    decode next to the chunks: bit-identical to the same three calls made one after another
    (store, decode, prefill); both stream forms match the oracle and store the same caches."""
    dev = device()
    c = mixed_case(611, [100, 0, 2000], [300, 64, 48], [50, 3000, 1, 999, 4096, 257], 16, 8, 128,
                   256)
    a, ka, va = run_mixed(c, 3, dev)
    side = torch.cuda.Stream(device=dev)  # default priority
    b, kb, vb = run_mixed(c, 3, dev, decode_stream=side)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ka), bits(kb)) and np.array_equal(bits(va), bits(vb))
    # the separate calls
    P, T = 3, c.total_q
    pt = int(c.cu_seqlens_q[P])
    kc, vc = bf16(c.k_cache, dev), bf16(c.v_cache, dev)
    q, kn, vn = bf16(c.q, dev), bf16(c.k_new, dev), bf16(c.v_new, dev)
    tables, ctx = i32(c.block_tables, dev), i32(c.context_lens, dev)
    pa.kvcache_store(kn, vn, i32(c.slot_mapping, dev), kc, vc)
    e = torch.empty((T, c.num_q_heads, c.head_dim), dtype=torch.float32, device=dev)
    pa.paged_decode(q[pt:], kc, vc, tables[P:], ctx[P:], c.scale, e[pt:])
    pa.paged_prefill(q[:pt], kn[:pt], vn[:pt], i32(c.cu_seqlens_q[:P + 1], dev), tables[:P],
                     ctx[:P], e[:pt], k_cache=kc, v_cache=vc, scale=c.scale,
                     max_q_len=int(c.q_lens[:P].max()))
    torch.cuda.synchronize()
    assert torch.equal(b, e)
    ref, _, _ = oracle_mixed(c)
    for got in (a, b):
        assert np.abs(as_f64(got) - ref).max() <= ATOL


def test_mixed_degenerate_mixes_equal_single_kind_calls():
    dev = device()
    c = mixed_case(612, [], [], [300, 17, 1025], 8, 2, 128, 16)
    out, _, _ = run_mixed(c, 0, dev)
    kc, vc = bf16(c.k_cache, dev), bf16(c.v_cache, dev)
    e = torch.empty_like(out)
    pa.paged_decode_append(bf16(c.q, dev), bf16(c.k_new, dev), bf16(c.v_new, dev),
                           i32(c.slot_mapping, dev), kc, vc, i32(c.block_tables, dev),
                           i32(c.context_lens, dev), c.scale, e)
    torch.cuda.synchronize()
    assert torch.equal(out, e)


@pytest.mark.parametrize("two_streams", [False, True], ids=["one_stream", "decode_stream"])
def test_mixed_chunk_reads_block_a_decode_row_fills(two_streams):
    """A chunk whose cached prefix ends with the block a decode row of the same step completes
    (prefix caching registers a block when its last token arrives): the chunk must read the
    decode row's new K/V, so every row is stored before any row attends, also when the decode
    rows run on a second stream.  The slot holds NaN until then."""
    dev = device()
    BS, Hq, Hkv, D, NB = 16, 8, 2, 128, 16
    rng = np.random.default_rng(613)
    from workloads import BF16_NAN, bf16_bits_from_f32

    def draw(*shape):
        return bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))

    A, X, Y, Z = 3, 9, 5, 12                     # physical blocks
    kc0 = np.full((NB, BS, Hkv, D), BF16_NAN, np.uint16)
    vc0 = kc0.copy()
    kc0[A], vc0[A] = draw(BS, Hkv, D), draw(BS, Hkv, D)
    kc0[X, :BS - 1], vc0[X, :BS - 1] = draw(BS - 1, Hkv, D), draw(BS - 1, Hkv, D)
    n = 20                                       # chunk: prefix of 32 tokens (blocks A, X)
    q = draw(n + 1, Hq, D)                       # chunk rows, then the decode row
    k_new, v_new = draw(n + 1, Hkv, D), draw(n + 1, Hkv, D)
    slots = np.array([Y * BS + j for j in range(BS)] + [Z * BS + j for j in range(n - BS)] +
                     [X * BS + BS - 1], np.int32)
    tables = np.full((2, 8), -1, np.int32)
    tables[0, :4] = [A, X, Y, Z]
    tables[1, :2] = [A, X]
    ctx = np.array([32 + n, 32], np.int32)
    scale = np.float32(1 / np.sqrt(D))
    okc, ovc = oracle.kvcache_store(k_new, v_new, slots, kc0, vc0)
    ref = oracle.paged_prefill(q, k_new, v_new, np.array([0, n, n + 1], np.int32), okc, ovc,
                               tables, ctx, scale)
    kc, vc = bf16(kc0, dev), bf16(vc0, dev)
    out = torch.empty((n + 1, Hq, D), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(device=dev) if two_streams else None  # default priority
    say(f"[mixed-shared-block] two streams: {two_streams}")
    pa.paged_attention_mixed(bf16(q, dev), bf16(k_new, dev), bf16(v_new, dev), i32(slots, dev),
                             i32(np.array([0, n], np.int32), dev), i32(tables, dev),
                             i32(ctx, dev), out, k_cache=kc, v_cache=vc, num_prefill_seqs=1,
                             prefill_tokens=n, max_prefill_q_len=n, scale=scale,
                             decode_stream=side)
    torch.cuda.synchronize()
    got = as_f64(out)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max()
    say(f"[mixed-shared-block] two streams {two_streams}: max|err| {err:.3e}")
    assert err <= ATOL
    assert np.array_equal(bits(kc), okc) and np.array_equal(bits(vc), ovc)
