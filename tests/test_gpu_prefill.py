"""HIP prefix-hit prefill vs the CPU oracle (max |err| <= 1e-2), on the prefill workload and on
edge cases: empty prefix, block-aligned and ragged prefixes, one-token chunks, chunks spanning
several token tiles, GQA groups that do not divide the 128-row tile, block sizes 1..1024."""
import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_86_amd as pa
from gpu_util import as_f64, bf16, bits, device, i32, say
from workloads import config, prefill_case

pytestmark = pytest.mark.gpu

ATOL = 1e-2


class PrefillOnDevice:
    def __init__(self, p, dev):
        self.p, self.dev = p, dev
        self.k_cache, self.v_cache = bf16(p.k_cache, dev), bf16(p.v_cache, dev)
        self.q, self.k_new, self.v_new = bf16(p.q, dev), bf16(p.k_new, dev), bf16(p.v_new, dev)
        self.cu, self.tables = i32(p.cu_seqlens_q, dev), i32(p.block_tables, dev)
        self.ctx, self.slots = i32(p.context_lens, dev), i32(p.slot_mapping, dev)

    def run(self, out_dtype=torch.float32, max_q_len=None):
        p = self.p
        out = torch.empty((p.total_q, p.num_q_heads, p.head_dim), dtype=out_dtype, device=self.dev)
        pa.paged_prefill(self.q, self.k_new, self.v_new, self.cu, self.tables, self.ctx, out,
                         k_cache=self.k_cache, v_cache=self.v_cache, scale=p.scale,
                         max_q_len=int(p.q_lens.max()) if max_q_len is None else max_q_len)
        return out


@functools.lru_cache(maxsize=None)
def workload5():
    say("[gen] workload 5")
    return config(5)


def test_prefill_workload():
    """The prefix-hit prefill workload, in the launch configuration the benchmark times."""
    dev = device()
    p = workload5()
    d = PrefillOnDevice(p, dev)
    say(f"[prefill] workload 5: B={p.batch} Tq={p.total_q} prefixes={p.prefix_lens.tolist()}")
    out32 = as_f64(d.run(torch.float32))
    out16 = as_f64(d.run(torch.bfloat16))
    say("[oracle] workload 5: all sequences")
    ref = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, np.float32(p.scale))
    err32 = float(np.abs(out32 - ref).max())
    err16 = float(np.abs(out16 - ref).max())
    say(f"[prefill] workload 5: max|err| fp32 {err32:.3e} bf16 {err16:.3e} over all {p.batch} "
        f"seqs ({p.total_q} rows)")
    assert err32 <= ATOL and err16 <= ATOL
    assert np.all(np.isfinite(out32))


def test_prefill_workload_chunk_store_bit_exact():
    """The store of the workload's 8192 chunk tokens: both whole pools bit for bit."""
    dev = device()
    p = workload5()
    d = PrefillOnDevice(p, dev)
    say(f"[store] workload 5: T={p.total_q}")
    pa.kvcache_store(d.k_new, d.v_new, d.slots, d.k_cache, d.v_cache)
    torch.cuda.synchronize()
    kc, vc = oracle.kvcache_store(p.k_new, p.v_new, p.slot_mapping, p.k_cache, p.v_cache)
    assert np.array_equal(bits(d.k_cache), kc)
    assert np.array_equal(bits(d.v_cache), vc)


SMALL = [
    # (D, BS, Hq, Hkv, prefix lengths, chunk lengths)
    (64, 16, 4, 2, [0, 20, 33], [5, 16, 9]),
    (128, 256, 16, 8, [0, 256, 300], [1, 64, 200]),
    (128, 16, 28, 4, [100, 0], [40, 19]),          # G = 7: 18 tokens per 128-row tile
    (64, 8, 8, 1, [7, 64], [130, 3]),              # G = 8: 16 tokens per tile, several tiles
    (128, 32, 2, 2, [513, 31], [129, 128]),        # G = 1: 128 tokens per tile
    (128, 1, 4, 4, [65, 0], [70, 1]),              # block size 1
    (64, 1024, 6, 2, [1100, 5], [300, 77]),        # block size 1024, G = 3
    (128, 64, 16, 1, [128, 191], [33, 65]),        # G = 16: 8 tokens per tile
    (64, 16, 4, 2, [17000, 16383, 5], [70, 2, 130]),  # more than the 1024 block ids staged in LDS
]


@pytest.mark.parametrize("case", SMALL, ids=[f"D{c[0]}_bs{c[1]}_h{c[2]}-{c[3]}_P{c[4]}" for c in SMALL])
def test_prefill_small_cases(case):
    dev = device()
    D, BS, Hq, Hkv, P, n = case
    p = prefill_case(4321 + D + BS + Hq, P, n, Hq, Hkv, D, BS)
    say(f"[prefill-small] D={D} BS={BS} Hq={Hq} Hkv={Hkv} P={P} n={n}")
    d = PrefillOnDevice(p, dev)
    out32 = as_f64(d.run(torch.float32))
    out16 = as_f64(d.run(torch.bfloat16))
    ref = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, np.float32(p.scale))
    assert np.abs(out32 - ref).max() <= ATOL
    assert np.abs(out16 - ref).max() <= ATOL
    # a chunk's first token with no prefix sees one key: its V, exactly
    G = Hq // Hkv
    for i in range(p.batch):
        if P[i] == 0:
            row = int(p.cu_seqlens_q[i])
            for h in range(Hq):
                assert np.array_equal(out32[row, h], oracle.bf16_to_f64(p.v_new[row, h // G]))


def test_prefill_grid_bound_and_determinism():
    """max_q_len larger than needed (extra tiles exit) gives bit-identical results, repeatably."""
    dev = device()
    p = prefill_case(55, [40, 300, 0], [100, 7, 250], 8, 2, 128, 16)
    d = PrefillOnDevice(p, dev)
    a = d.run(torch.float32)
    b = d.run(torch.float32, max_q_len=p.total_q)
    c = d.run(torch.float32)
    assert torch.equal(a, b) and torch.equal(a, c)


def test_prefill_last_row_equals_decode():
    """The last chunk token's output equals a decode step over the stored chunk."""
    dev = device()
    p = prefill_case(56, [90, 0, 513], [37, 64, 1], 8, 4, 128, 16, num_blocks=64)
    d = PrefillOnDevice(p, dev)
    out = d.run(torch.float32)
    pa.kvcache_store(d.k_new, d.v_new, d.slots, d.k_cache, d.v_cache)
    last = (p.cu_seqlens_q[1:] - 1).astype(np.int64)
    q_last = d.q[torch.from_numpy(last).to(dev)].contiguous()
    dec = torch.empty((p.batch, p.num_q_heads, p.head_dim), dtype=torch.float32, device=dev)
    pa.paged_decode(q_last, d.k_cache, d.v_cache, d.tables, d.ctx, p.scale, dec)
    assert (out[torch.from_numpy(last).to(dev)] - dec).abs().max().item() <= 2e-3


def test_prefill_item_order_does_not_change_results():
    """Items run longest first up to 4096 (token tile, sequence) items and in index order
    beyond: a max_q_len that takes the grid past that limit (the extra tiles exit) gives
    bit-identical outputs."""
    dev = device()
    rng = np.random.default_rng(57)
    B = 260
    p = prefill_case(57, rng.integers(0, 41, B), rng.integers(1, 4, B), 16, 1, 64, 16)
    d = PrefillOnDevice(p, dev)
    tt_tokens = 128 // (p.num_q_heads // p.num_kv_heads)
    big = p.total_q
    assert B * ((int(p.q_lens.max()) + tt_tokens - 1) // tt_tokens) <= 4096
    assert B * ((big + tt_tokens - 1) // tt_tokens) > 4096
    say(f"[prefill-order] B={B} max_q_len {int(p.q_lens.max())} vs {big}")
    ranked = d.run(torch.float32)
    indexed = d.run(torch.float32, max_q_len=big)
    assert torch.equal(ranked, indexed)
    ref = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, np.float32(p.scale))
    assert np.abs(as_f64(ranked) - ref).max() <= ATOL


def test_prefill_many_sequences():
    """4100 short chunks (more items than the ranked order takes) against the oracle."""
    dev = device()
    rng = np.random.default_rng(58)
    B = 4100
    P = rng.integers(0, 41, B)
    n = rng.integers(1, 4, B)
    p = prefill_case(58, P, n, 2, 1, 64, 16)
    say(f"[prefill-many] B={B} Tq={p.total_q}")
    out = as_f64(PrefillOnDevice(p, dev).run(torch.float32))
    ref = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, np.float32(p.scale))
    assert np.abs(out - ref).max() <= ATOL
