"""FP8 (E4M3) prefix-hit prefill, HIP path vs the CPU oracle: the pools are quantized and the
chunk's own tokens stored by the library's FP8 store (the codes the kernel reads are compared bit
for bit with the oracle's), every key is read through the block table, outputs within 1e-2."""
import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_86_amd as pa
from gpu_util import as_f64, bf16, device, i32, say
from workloads import config, prefill_case

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def codes(t) -> np.ndarray:
    return t.cpu().numpy().astype(np.uint8)


class Fp8PrefillOnDevice:
    """A prefill chunk over FP8 pools: the bf16 pools quantized, then the chunk stored."""

    def __init__(self, p, dev, k_scale, v_scale):
        self.p, self.dev, self.ks, self.vs = p, dev, k_scale, v_scale
        NB, BS, Hkv, D = p.k_cache.shape
        self.k8 = torch.empty((NB, BS, Hkv, D), dtype=torch.uint8, device=dev)
        self.v8 = torch.empty_like(self.k8)
        every = i32(np.arange(NB * BS, dtype=np.int32), dev)
        pa.kvcache_store_fp8(bf16(p.k_cache.reshape(NB * BS, Hkv, D), dev),
                             bf16(p.v_cache.reshape(NB * BS, Hkv, D), dev), every, self.k8, self.v8,
                             k_scale, v_scale)
        pa.kvcache_store_fp8(bf16(p.k_new, dev), bf16(p.v_new, dev), i32(p.slot_mapping, dev),
                             self.k8, self.v8, k_scale, v_scale)
        self.q, self.cu = bf16(p.q, dev), i32(p.cu_seqlens_q, dev)
        self.tables, self.ctx = i32(p.block_tables, dev), i32(p.context_lens, dev)

    def run(self, out_dtype=torch.float32, max_q_len=None):
        p = self.p
        out = torch.empty((p.total_q, p.num_q_heads, p.head_dim), dtype=out_dtype, device=self.dev)
        pa.paged_prefill_fp8(self.q, self.cu, self.tables, self.ctx, out, k_cache=self.k8,
                             v_cache=self.v8, scale=p.scale, k_scale=self.ks, v_scale=self.vs,
                             max_q_len=int(p.q_lens.max()) if max_q_len is None else max_q_len)
        return out

    def oracle_pools(self, blocks):
        """The oracle's FP8 pools on the given physical blocks (zero codes elsewhere), chunk
        stored.  ``oracle.quantize`` is elementwise: it is evaluated once on every bf16 pattern
        and the pools are looked up in that table."""
        p = self.p
        every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        with np.errstate(over="ignore", invalid="ignore"):
            lut_k, lut_v = oracle.quantize(every, self.ks), oracle.quantize(every, self.vs)
        kc8 = np.zeros(p.k_cache.shape, np.uint8)
        vc8 = np.zeros(p.v_cache.shape, np.uint8)
        kc8[blocks] = lut_k[p.k_cache[blocks]]
        vc8[blocks] = lut_v[p.v_cache[blocks]]
        return oracle.kvcache_store_fp8(p.k_new, p.v_new, p.slot_mapping, kc8, vc8, self.ks, self.vs)


def check(d, label):
    """Every chunk row against the oracle; the codes on every block the tables name are
    compared bit for bit with the oracle's first."""
    p = d.p
    out32 = as_f64(d.run(torch.float32))
    out16 = as_f64(d.run(torch.bfloat16))
    blocks = np.unique(p.block_tables[p.block_tables >= 0])
    kc8, vc8 = d.oracle_pools(blocks)
    sel = torch.as_tensor(blocks, dtype=torch.int64, device=d.dev)
    assert np.array_equal(codes(d.k8[sel]), kc8[blocks])
    assert np.array_equal(codes(d.v8[sel]), vc8[blocks])
    ref = oracle.paged_prefill_fp8(p.q, p.cu_seqlens_q, kc8, vc8, p.block_tables,
                                   p.context_lens, np.float32(p.scale), d.ks, d.vs)
    err32 = float(np.abs(out32 - ref).max())
    err16 = float(np.abs(out16 - ref).max())
    say(f"[prefill-fp8] {label}: max|err| fp32 {err32:.3e} bf16 {err16:.3e} over all "
        f"{p.batch} seqs")
    assert err32 <= ATOL and err16 <= ATOL
    assert np.all(np.isfinite(out32))
    return out32, vc8


def test_prefill_fp8_workload():
    """The prefix-hit prefill workload on FP8 pools (amax/448 scales)."""
    dev = device()
    p = config(5)
    x = oracle.bf16_to_f64(p.k_new)
    ks = float(np.float32(np.abs(x).max() / oracle.E4M3_MAX))
    vs = float(np.float32(np.abs(oracle.bf16_to_f64(p.v_new)).max() / oracle.E4M3_MAX))
    say(f"[prefill-fp8] workload 5: k_scale={ks:.4g} v_scale={vs:.4g}")
    d = Fp8PrefillOnDevice(p, dev, ks, vs)
    check(d, "workload 5")


SMALL = [
    # (D, BS, Hq, Hkv, prefix lengths, chunk lengths)
    (64, 16, 4, 2, [0, 20, 33], [5, 16, 9]),
    (128, 256, 16, 8, [0, 256, 300], [1, 64, 200]),
    (128, 16, 28, 4, [100, 0], [40, 19]),          # G = 7
    (64, 8, 8, 1, [7, 64], [130, 3]),              # G = 8, several token tiles
    (128, 32, 2, 2, [513, 31], [129, 128]),        # G = 1
    (128, 1, 4, 4, [65, 0], [70, 1]),              # block size 1
    (64, 1024, 6, 2, [1100, 5], [300, 77]),        # block size 1024, G = 3
    (64, 16, 4, 2, [17000, 16383, 5], [70, 2, 130]),  # more than the 1024 block ids staged in LDS
]


@pytest.mark.parametrize("case", SMALL, ids=[f"D{c[0]}_bs{c[1]}_h{c[2]}-{c[3]}_P{c[4]}" for c in SMALL])
def test_prefill_fp8_small_cases(case):
    dev = device()
    D, BS, Hq, Hkv, P, n = case
    p = prefill_case(9753 + D + BS + Hq, P, n, Hq, Hkv, D, BS)
    say(f"[prefill-fp8-small] D={D} BS={BS} Hq={Hq} Hkv={Hkv} P={P} n={n}")
    d = Fp8PrefillOnDevice(p, dev, 0.0125, 0.02)
    out32, vc8 = check(d, f"D{D} bs{BS} h{Hq}/{Hkv}")
    # a chunk's first token with no prefix sees one key: code(v) * v_scale, exactly
    G = Hq // Hkv
    for i in range(p.batch):
        if P[i] == 0:
            row = int(p.cu_seqlens_q[i])
            blk, off = divmod(int(p.slot_mapping[row]), BS)
            vrow = np.float32(oracle.e4m3_decode(vc8[blk, off]) * np.float32(d.vs))
            for h in range(Hq):
                assert np.array_equal(out32[row, h], vrow[h // G].astype(np.float64))


def test_prefill_fp8_last_row_equals_fp8_decode():
    """The last chunk token's output equals an FP8 decode step over the same pools."""
    dev = device()
    p = prefill_case(57, [90, 0, 513], [37, 64, 1], 8, 4, 128, 16, num_blocks=64)
    d = Fp8PrefillOnDevice(p, dev, 0.0125, 0.02)
    out = d.run(torch.float32)
    last = torch.from_numpy((p.cu_seqlens_q[1:] - 1).astype(np.int64)).to(dev)
    dec = torch.empty((p.batch, p.num_q_heads, p.head_dim), dtype=torch.float32, device=dev)
    pa.paged_decode_fp8(d.q[last].contiguous(), d.k8, d.v8, d.tables, d.ctx, p.scale, d.ks, d.vs,
                        dec)
    assert (out[last] - dec).abs().max().item() <= 2e-3
    assert torch.equal(out, d.run(torch.float32))  # deterministic


def test_prefill_fp8_scales_fold_exactly():
    """Powers of two moved between the softmax scale and k_scale leave the outputs unchanged;
    doubling v_scale doubles them exactly."""
    dev = device()
    p = prefill_case(58, [30, 0], [20, 9], 4, 2, 64, 16)
    d = Fp8PrefillOnDevice(p, dev, 0.0125, 0.02)
    base = d.run(torch.float32)
    out = torch.empty_like(base)
    pa.paged_prefill_fp8(d.q, d.cu, d.tables, d.ctx, out, k_cache=d.k8, v_cache=d.v8,
                         scale=p.scale / 2, k_scale=d.ks * 2, v_scale=d.vs, max_q_len=20)
    assert torch.equal(out, base)
    pa.paged_prefill_fp8(d.q, d.cu, d.tables, d.ctx, out, k_cache=d.k8, v_cache=d.v8,
                         scale=p.scale, k_scale=d.ks, v_scale=d.vs * 2, max_q_len=20)
    assert torch.equal(out, base * 2)
