"""FP8 (OCP E4M3) KV cache, HIP path vs the CPU oracle: the quantizing store bit-exact
(every bfloat16 bit pattern, several scales, workload shapes) and decode on an FP8 pool
within 1e-2 of attention on the dequantized keys and values."""
import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_86_amd as pa
from gpu_util import as_f64, bf16, device, i32, say
from workloads import config, decode_case

pytestmark = pytest.mark.gpu

ATOL = 1e-2

# A power of two, the typical amax/448 of N(0, 1) data, non-dyadic values, and scales that
# push almost everything into saturation (tiny) or into the subnormal codes and zero (huge).
SCALES = [1.0, 0.0107421875, 0.3, 0.017, 2.0 ** -12, 1e-30, 3.7e4, 1e6]


def u8(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def codes(t) -> np.ndarray:
    return t.cpu().numpy().astype(np.uint8)


@pytest.mark.parametrize("ks", SCALES)
def test_store_fp8_every_bf16_pattern(ks):
    """All 65536 bf16 bit patterns (NaNs, infinities, subnormals, signed zeros) through the store."""
    dev = device()
    D, Hkv = 128, 2
    T = 65536 // (Hkv * D)
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    k = allbits.reshape(T, Hkv, D)
    v = allbits[::-1].reshape(T, Hkv, D)
    vs = 1.0 / ks
    NB, BS = T // 8 + 3, 8
    perm = np.random.default_rng(5).permutation(NB * BS)[:T].astype(np.int32)
    say(f"[fp8-store] every bf16 pattern, k_scale={ks} v_scale={vs}")
    kc = torch.full((NB, BS, Hkv, D), 0x5A, dtype=torch.uint8, device=dev)
    vc = torch.full((NB, BS, Hkv, D), 0xA5, dtype=torch.uint8, device=dev)
    pa.kvcache_store_fp8(bf16(k, dev), bf16(v, dev), i32(perm, dev), kc, vc, ks, vs)
    want_k, want_v = oracle.kvcache_store_fp8(
        k, v, perm, np.full((NB, BS, Hkv, D), 0x5A, np.uint8),
        np.full((NB, BS, Hkv, D), 0xA5, np.uint8), ks, vs)
    got_k, got_v = codes(kc), codes(vc)
    bad = np.nonzero(got_k.reshape(-1) != want_k.reshape(-1))[0]
    if bad.size:
        i = int(bad[0])
        flat_slot, within = divmod(i, Hkv * D)
        t = int(np.nonzero(perm == flat_slot)[0][0])
        x = int(k.reshape(T, -1)[t, within])
        say(f"[fp8-store] first K mismatch: bf16 0x{x:04x} -> gpu 0x{got_k.reshape(-1)[i]:02x} "
            f"oracle 0x{want_k.reshape(-1)[i]:02x} ({bad.size} mismatches)")
    assert bad.size == 0
    assert np.array_equal(got_v, want_v)


@functools.lru_cache(maxsize=None)
def workload(cfg_id):
    say(f"[gen] workload {cfg_id}")
    return config(cfg_id)


def amax_scale(bits) -> float:
    """Per-tensor scale amax / 448 of the finite values (a test input, not library arithmetic)."""
    x = oracle.bf16_to_f64(bits)
    return float(np.float32(np.nanmax(np.abs(x[np.isfinite(x)])) / oracle.E4M3_MAX))


class Fp8Pool:
    """A decode workload with its pools quantized on the GPU by the library's own store."""

    def __init__(self, c, dev, k_scale, v_scale):
        self.c, self.dev = c, dev
        self.ks, self.vs = k_scale, v_scale
        NB, BS, Hkv, D = c.k_cache.shape
        self.k_cache = torch.empty((NB, BS, Hkv, D), dtype=torch.uint8, device=dev)
        self.v_cache = torch.empty_like(self.k_cache)
        every = np.arange(NB * BS, dtype=np.int32)
        pa.kvcache_store_fp8(bf16(c.k_cache.reshape(NB * BS, Hkv, D), dev),
                             bf16(c.v_cache.reshape(NB * BS, Hkv, D), dev), i32(every, dev),
                             self.k_cache, self.v_cache, k_scale, v_scale)
        self.q = bf16(c.q, dev)
        self.tables = i32(c.block_tables, dev)
        self.ctx = i32(c.context_lens, dev)
        pa.kvcache_store_fp8(bf16(c.k_new, dev), bf16(c.v_new, dev), i32(c.slot_mapping, dev),
                             self.k_cache, self.v_cache, k_scale, v_scale)

    def oracle_pools(self, blocks):
        """The oracle's FP8 pools on the given physical blocks (zero codes elsewhere).

        ``oracle.quantize`` is elementwise, so it is evaluated once on every bf16 pattern and
        the pools are looked up in that table (large pools would not fit its float64
        temporaries)."""
        c = self.c
        every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        with np.errstate(over="ignore", invalid="ignore"):
            lut_k, lut_v = oracle.quantize(every, self.ks), oracle.quantize(every, self.vs)
        kc8 = np.zeros(c.k_cache.shape, np.uint8)
        vc8 = np.zeros(c.v_cache.shape, np.uint8)
        kc8[blocks] = lut_k[c.k_cache[blocks]]
        vc8[blocks] = lut_v[c.v_cache[blocks]]
        return oracle.kvcache_store_fp8(c.k_new, c.v_new, c.slot_mapping, kc8, vc8, self.ks,
                                        self.vs)

    def decode(self, out_dtype=torch.float32, tables=None, k_cache=None, v_cache=None,
               workspace=None):
        c = self.c
        out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=out_dtype, device=self.dev)
        pa.paged_decode_fp8(self.q, self.k_cache if k_cache is None else k_cache,
                            self.v_cache if v_cache is None else v_cache,
                            self.tables if tables is None else tables, self.ctx, c.scale,
                            self.ks, self.vs, out, workspace=workspace)
        return out


def check_decode(d: Fp8Pool, label=""):
    """Every sequence against the oracle; the GPU's codes on every block the tables name are
    compared bit for bit with the oracle's first."""
    c = d.c
    out32 = as_f64(d.decode(torch.float32))
    out16 = as_f64(d.decode(torch.bfloat16))
    blocks = np.unique(c.block_tables[c.block_tables >= 0])
    kc8, vc8 = d.oracle_pools(blocks)
    sel = torch.as_tensor(blocks, dtype=torch.int64, device=d.dev)
    assert np.array_equal(codes(d.k_cache[sel]), kc8[blocks])
    assert np.array_equal(codes(d.v_cache[sel]), vc8[blocks])
    ref = oracle.paged_decode_fp8(c.q, kc8, vc8, c.block_tables, c.context_lens,
                                  np.float32(c.scale), d.ks, d.vs)
    e32 = np.abs(out32 - ref).max()
    e16 = np.abs(out16 - ref).max()
    say(f"[fp8-decode] {label}: max|err| fp32 {e32:.3e} bf16 {e16:.3e} over all {c.batch} seqs")
    assert e32 <= ATOL and e16 <= ATOL
    assert np.all(np.isfinite(out32))
    d.ref = ref
    return out32, kc8, vc8


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_decode_fp8_workload(cfg_id):
    dev = device()
    c = workload(cfg_id)
    ks, vs = amax_scale(c.k_cache), amax_scale(c.v_cache)
    say(f"[fp8-decode] workload {cfg_id}: B={c.batch} k_scale={ks:.4g} v_scale={vs:.4g}")
    d = Fp8Pool(c, dev, ks, vs)
    check_decode(d, f"workload {cfg_id}")
    # the fused quantizing store + decode (the timed FP8 step): the pools already hold the new
    # rows, which it writes again (same slots, same codes), and every output row is checked
    kb, vb = d.k_cache.clone(), d.v_cache.clone()
    for dt in (torch.float32, torch.bfloat16):
        out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=dt, device=dev)
        pa.paged_decode_append_fp8(d.q, bf16(c.k_new, dev), bf16(c.v_new, dev),
                                   i32(c.slot_mapping, dev), d.k_cache, d.v_cache, d.tables,
                                   d.ctx, c.scale, ks, vs, out)
        err = np.abs(as_f64(out) - d.ref).max()
        say(f"[fp8-append] workload {cfg_id} {dt}: max|err| {err:.3e} over all {c.batch} seqs")
        assert err <= ATOL
    assert torch.equal(kb, d.k_cache) and torch.equal(vb, d.v_cache)


SMALL = [
    # (D, BS, Hq, Hkv, context lengths)
    (64, 16, 2, 1, [17, 64, 200, 255, 513]),
    (64, 1, 4, 4, [1, 2, 3, 70]),
    (64, 8, 8, 2, [0, 1, 7, 8, 9, 0, 63, 64, 65]),
    (128, 16, 28, 4, [512, 1, 300, 1024]),          # 7 heads per KV head (MFMA kernel)
    (128, 256, 16, 8, [1, 255, 256, 257, 511, 512, 513, 4096]),
    (128, 32, 5, 1, [129, 33, 2000]),               # 5 heads (MFMA)
    (128, 16, 32, 4, [100, 1, 777]),                # 8 heads (MFMA)
    (64, 64, 16, 1, [5, 300, 1024]),                # 16 heads: one MFMA workgroup
    (128, 16, 20, 1, [700, 1, 257]),                # 20 heads: two MFMA sub-groups of 10
    (64, 32, 32, 1, [64, 1000, 3]),                 # 32 heads: two MFMA sub-groups of 16
    (128, 1024, 2, 2, [3000, 1025]),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"D{c[0]}_bs{c[1]}_h{c[2]}-{c[3]}" for c in SMALL])
def test_decode_fp8_small_cases(case):
    dev = device()
    D, BS, Hq, Hkv, ctx = case
    c = decode_case(4321 + D + BS + Hq, ctx, Hq, Hkv, D, BS, nb_factor=1.4)
    say(f"[fp8-decode-small] D={D} BS={BS} Hq={Hq} Hkv={Hkv} ctx={ctx}")
    d = Fp8Pool(c, dev, 0.0125, 0.02)
    out32, kc8, vc8 = check_decode(d, label=f"D{D} bs{BS}")
    G = Hq // Hkv
    for i, n in enumerate(ctx):
        if n == 0:
            assert np.all(out32[i] == 0)
        if n == 1:  # one key: the output is that token's V, code * v_scale rounded to fp32
            blk, off = divmod(int(c.slot_mapping[i]), BS)
            vrow = np.float32(oracle.e4m3_decode(vc8[blk, off]) * np.float32(d.vs))
            for h in range(Hq):
                assert np.array_equal(out32[i, h], vrow[h // G].astype(np.float64))


def test_decode_fp8_block_permutation_bit_identical():
    dev = device()
    c = decode_case(91, [300, 1, 513, 40, 1024], 8, 2, 128, 16, nb_factor=1.5)
    d = Fp8Pool(c, dev, 0.0125, 0.02)
    a = d.decode(torch.float32)
    perm = np.random.default_rng(92).permutation(c.num_blocks)
    kc, vc = codes(d.k_cache), codes(d.v_cache)
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm] = kc
    vp[perm] = vc
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1)
    b = d.decode(torch.float32, tables=i32(bt, dev), k_cache=u8(kp, dev), v_cache=u8(vp, dev))
    assert torch.equal(a, b)
    assert torch.equal(a, d.decode(torch.float32))  # deterministic


def test_decode_fp8_scales_fold_exactly():
    """Scaling k_scale by 2 and the softmax scale by 1/2 leaves the scores, hence outputs, unchanged;
    scaling v_scale by 2 doubles the outputs exactly (powers of two are exact in fp32)."""
    dev = device()
    c = decode_case(93, [700, 64, 1], 8, 4, 64, 16, nb_factor=1.3)
    d = Fp8Pool(c, dev, 0.0125, 0.02)
    base = d.decode(torch.float32)
    out = torch.empty_like(base)
    pa.paged_decode_fp8(d.q, d.k_cache, d.v_cache, d.tables, d.ctx, c.scale / 2, d.ks * 2, d.vs,
                        out)
    assert torch.equal(out, base)
    pa.paged_decode_fp8(d.q, d.k_cache, d.v_cache, d.tables, d.ctx, c.scale, d.ks, d.vs * 2, out)
    assert torch.equal(out, base * 2)


@pytest.mark.parametrize("case", SMALL[:6] + [(64, 16, 4, 2, [512, 513, 1025, 1, 0])],
                         ids=lambda c: f"D{c[0]}_bs{c[1]}_h{c[2]}-{c[3]}")
def test_decode_append_fp8(case):
    """Fused quantizing store + decode equals store_fp8 then decode_fp8 (caches bit-exact)."""
    dev = device()
    D, BS, Hq, Hkv, ctx = case
    c = decode_case(8642 + D + BS + Hq, ctx, Hq, Hkv, D, BS, nb_factor=1.4)
    say(f"[fp8-append] D={D} BS={BS} Hq={Hq} Hkv={Hkv} ctx={ctx}")
    ks, vs = 0.0125, 0.02
    NB, _, _, _ = c.k_cache.shape
    kc = torch.empty((NB, BS, Hkv, D), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    every = np.arange(NB * BS, dtype=np.int32)
    pa.kvcache_store_fp8(bf16(c.k_cache.reshape(NB * BS, Hkv, D), dev),
                         bf16(c.v_cache.reshape(NB * BS, Hkv, D), dev), i32(every, dev), kc, vc,
                         ks, vs)
    out = torch.empty((c.batch, Hq, D), dtype=torch.float32, device=dev)
    pa.paged_decode_append_fp8(bf16(c.q, dev), bf16(c.k_new, dev), bf16(c.v_new, dev),
                               i32(c.slot_mapping, dev), kc, vc, i32(c.block_tables, dev),
                               i32(c.context_lens, dev), c.scale, ks, vs, out)
    kc8, vc8 = oracle.kvcache_store_fp8(c.k_new, c.v_new, c.slot_mapping,
                                        oracle.quantize(c.k_cache, ks),
                                        oracle.quantize(c.v_cache, vs), ks, vs)
    assert np.array_equal(codes(kc), kc8) and np.array_equal(codes(vc), vc8)
    ref = oracle.paged_decode_fp8(c.q, kc8, vc8, c.block_tables, c.context_lens,
                                  np.float32(c.scale), ks, vs)
    got = as_f64(out)
    err = np.abs(got - ref).max()
    say(f"[fp8-append] max|err| fp32 {err:.3e}")
    assert err <= ATOL
    G = Hq // Hkv
    for i, n in enumerate(ctx):
        if n == 0:
            assert np.all(got[i] == 0)
        if n == 1:
            blk, off = divmod(int(c.slot_mapping[i]), BS)
            vrow = np.float32(oracle.e4m3_decode(vc8[blk, off]) * np.float32(vs))
            for h in range(Hq):
                assert np.array_equal(got[i, h], vrow[h // G].astype(np.float64))


def test_decode_fp8_long_splits():
    """128 x 16/8 heads at block 256: on an FP8 pool every context of more than one short
    split takes splits of 512 tokens (one-split contexts and every boundary around 1, 2, 8, 9
    and 16 short splits), plain and fused store."""
    dev = device()
    S = 256
    edges = [1, 2, S - 1, S, S + 1, 8 * S - 1, 8 * S, 8 * S + 1, 9 * S, 9 * S + 1, 16 * S - 1,
             16 * S, 0, 2 * S, 2 * S + 1, 3 * S - 1]
    rng = np.random.default_rng(4444)
    ctx = edges + [int(x) for x in rng.integers(1, 16 * S, 128 - len(edges), endpoint=True)]
    c = decode_case(4444, ctx, 16, 8, 128, 256, nb_factor=1.2, max_blocks_per_seq=16)
    say(f"[fp8-long] B=128 ctx max {int(c.context_lens.max())}")
    check_decode(Fp8Pool(c, dev, 0.0125, 0.02), label="long splits")
    ks, vs = 0.0125, 0.02
    NB = c.k_cache.shape[0]
    kc = torch.empty((NB, 256, 8, 128), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    every = np.arange(NB * 256, dtype=np.int32)
    pa.kvcache_store_fp8(bf16(c.k_cache.reshape(NB * 256, 8, 128), dev),
                         bf16(c.v_cache.reshape(NB * 256, 8, 128), dev), i32(every, dev), kc, vc,
                         ks, vs)
    out = torch.empty((128, 16, 128), dtype=torch.float32, device=dev)
    pa.paged_decode_append_fp8(bf16(c.q, dev), bf16(c.k_new, dev), bf16(c.v_new, dev),
                               i32(c.slot_mapping, dev), kc, vc, i32(c.block_tables, dev),
                               i32(c.context_lens, dev), c.scale, ks, vs, out)
    kc8, vc8 = oracle.kvcache_store_fp8(c.k_new, c.v_new, c.slot_mapping,
                                        oracle.quantize(c.k_cache, ks),
                                        oracle.quantize(c.v_cache, vs), ks, vs)
    assert np.array_equal(codes(kc), kc8) and np.array_equal(codes(vc), vc8)
    ref = oracle.paged_decode_fp8(c.q, kc8, vc8, c.block_tables, c.context_lens,
                                  np.float32(c.scale), ks, vs)
    err = np.abs(as_f64(out) - ref).max()
    say(f"[fp8-long] fused store: max|err| {err:.3e}")
    assert err <= ATOL


def test_decode_fp8_mfma_long_splits():
    """7 query heads per KV head on an FP8 pool, 128 sequences with 8,192-token tables at block
    16: the MFMA kernel's 2,048-token splits, every boundary of both split lengths, plain and
    fused store, every sequence against the oracle."""
    dev = device()
    S, L = 256, 2048
    edges = [1, 2, S - 1, S, S + 1, L - 1, L, L + 1, 2 * L, 2 * L + 1, 4 * L - 1, 4 * L, 0, 33]
    rng = np.random.default_rng(5252)
    ctx = edges + [int(x) for x in rng.integers(1, 4 * L, 128 - len(edges), endpoint=True)]
    c = decode_case(5252, ctx, 28, 4, 128, 16, nb_factor=1.1, max_blocks_per_seq=4 * L // 16)
    say(f"[fp8-mfma-long] B=128 ctx max {int(c.context_lens.max())}")
    check_decode(Fp8Pool(c, dev, 0.0125, 0.02), label="mfma long splits")
    ks, vs = 0.0125, 0.02
    NB = c.k_cache.shape[0]
    kc = torch.empty((NB, 16, 4, 128), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    every = np.arange(NB * 16, dtype=np.int32)
    pa.kvcache_store_fp8(bf16(c.k_cache.reshape(NB * 16, 4, 128), dev),
                         bf16(c.v_cache.reshape(NB * 16, 4, 128), dev), i32(every, dev), kc, vc,
                         ks, vs)
    out = torch.empty((128, 28, 128), dtype=torch.float32, device=dev)
    pa.paged_decode_append_fp8(bf16(c.q, dev), bf16(c.k_new, dev), bf16(c.v_new, dev),
                               i32(c.slot_mapping, dev), kc, vc, i32(c.block_tables, dev),
                               i32(c.context_lens, dev), c.scale, ks, vs, out)
    kc8, vc8 = oracle.kvcache_store_fp8(c.k_new, c.v_new, c.slot_mapping,
                                        oracle.quantize(c.k_cache, ks),
                                        oracle.quantize(c.v_cache, vs), ks, vs)
    assert np.array_equal(codes(kc), kc8) and np.array_equal(codes(vc), vc8)
    ref = oracle.paged_decode_fp8(c.q, kc8, vc8, c.block_tables, c.context_lens,
                                  np.float32(c.scale), ks, vs)
    err = np.abs(as_f64(out) - ref).max()
    say(f"[fp8-mfma-long] fused store: max|err| {err:.3e}")
    assert err <= ATOL


FP8_MAX_CASES = [(2, 1), (7, 1)]  # VALU (long splits: 8 sequences x 128 slots), MFMA


@pytest.mark.parametrize("Hq,Hkv", FP8_MAX_CASES, ids=[f"h{a}-{b}" for a, b in FP8_MAX_CASES])
def test_decode_fp8_max_context(Hq, Hkv):
    """FP8 pools at the longest context one decode call takes (256 short splits of 256 tokens
    at head_dim 128, a table exactly that wide), next to one-token and short contexts.  On
    the VALU kernel 8 sequences make the grid large enough for splits of twice the length."""
    dev = device()
    maxc, BS = 256 * 256, 256
    ctx = [maxc, 1, maxc - 1, 300] + ([4097, 0, 513, 2] if Hq == 2 else [])
    c = decode_case(9200 + Hq + Hkv, ctx, Hq, Hkv, 128, BS, nb_factor=1.05,
                    max_blocks_per_seq=maxc // BS)
    if Hq == 2:  # 8 sequences x 128 long-split slots: long splits are on, so the plan at 8
        # needs less than 7 sequences with short splits (the size is the most of either)
        ws = [pa.decode_fp8_workspace_bytes(b, 2, 1, 128, BS, maxc // BS) for b in (6, 7, 8)]
        assert ws[0] < ws[1] == ws[2]
    say(f"[fp8-max] h={Hq}/{Hkv} ctx={ctx}")
    check_decode(Fp8Pool(c, dev, 0.0125, 0.02), label=f"max context h{Hq}/{Hkv}")
