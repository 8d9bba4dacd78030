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


def test_mixed_second_stream_bit_identical():
    dev = device()
    c = mixed_case(611, [100, 0, 2000], [300, 64, 48], [50, 3000, 1, 999, 4096, 257], 16, 8, 128,
                   256)
    a, ka, va = run_mixed(c, 3, dev)
    side = torch.cuda.Stream(device=dev)  # default priority
    b, kb, vb = run_mixed(c, 3, dev, decode_stream=side)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert np.array_equal(bits(ka), bits(kb)) and np.array_equal(bits(va), bits(vb))
    ref, _, _ = oracle_mixed(c)
    assert np.abs(as_f64(b) - ref).max() <= ATOL


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
