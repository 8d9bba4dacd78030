"""HIP path vs the CPU oracle: KV store and block-table un-page bit-exact, paged decode within
1e-2 (bf16 inputs, fp32 accumulation), on the five workloads and on small edge cases."""
import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_86_amd as pa
from gpu_util import DecodeOnDevice, as_f64, bf16, bits, device, i32, say
from workloads import config, decode_case

pytestmark = pytest.mark.gpu

ATOL = 1e-2  # max |gpu - oracle| for attention outputs, bf16 inputs with fp32 accumulation


@functools.lru_cache(maxsize=None)
def workload(cfg_id):
    say(f"[gen] workload {cfg_id}")
    return config(cfg_id)


@functools.lru_cache(maxsize=None)
def oracle_store(cfg_id):
    c = workload(cfg_id)
    return oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)


@functools.lru_cache(maxsize=None)
def oracle_decode(cfg_id):
    """The oracle's outputs for every sequence of a workload (after its store)."""
    c = workload(cfg_id)
    kc, vc = oracle_store(cfg_id)
    say(f"[oracle] workload {cfg_id}: all {c.batch} sequences")
    return oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_store_bit_exact(cfg_id):
    dev = device()
    c = workload(cfg_id)
    say(f"[store] workload {cfg_id}: T={c.batch}")
    d = DecodeOnDevice(c, dev)
    d.store()
    torch.cuda.synchronize()
    kc, vc = oracle_store(cfg_id)
    assert np.array_equal(bits(d.k_cache), kc)
    assert np.array_equal(bits(d.v_cache), vc)


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_gather_bit_exact(cfg_id):
    dev = device()
    c = workload(cfg_id)
    kc, vc = oracle_store(cfg_id)
    say(f"[gather] workload {cfg_id}")
    cu = np.zeros(c.batch + 1, np.int32)
    cu[1:] = np.cumsum(c.context_lens)
    total = int(cu[-1])
    for name, pool in (("k", kc), ("v", vc)):
        out = torch.empty((total, c.num_kv_heads, c.head_dim), dtype=torch.bfloat16, device=dev)
        pa.paged_gather(bf16(pool, dev), i32(c.block_tables, dev), i32(c.context_lens, dev),
                        i32(cu, dev), int(c.context_lens.max()), out)
        got = bits(out)
        for i in range(c.batch):
            want = oracle.unpage(pool, c.block_tables[i], int(c.context_lens[i]))
            assert np.array_equal(got[cu[i]:cu[i + 1]], want), (name, i)


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_decode_workload(cfg_id):
    """Store + decode in the launch configuration the benchmark times; fp32 and bf16 outputs."""
    dev = device()
    c = workload(cfg_id)
    d = DecodeOnDevice(c, dev)
    say(f"[decode] workload {cfg_id}: B={c.batch} Hq={c.num_q_heads} Hkv={c.num_kv_heads}")
    d.store()
    out32 = as_f64(d.decode(torch.float32))
    out16 = as_f64(d.decode(torch.bfloat16))
    ref = oracle_decode(cfg_id)
    err32 = np.abs(out32 - ref).max()
    err16 = np.abs(out16 - ref).max()
    say(f"[decode] workload {cfg_id}: max|err| fp32 {err32:.3e} bf16 {err16:.3e} over all "
        f"{c.batch} seqs")
    assert err32 <= ATOL and err16 <= ATOL
    assert np.all(np.isfinite(out32))


SMALL = [
    # (D, BS, Hq, Hkv, context lengths)
    (64, 16, 2, 1, [17, 64, 200, 255]),
    (64, 1, 4, 4, [1, 2, 3, 70]),
    (64, 8, 8, 2, [0, 1, 7, 8, 9, 0, 63, 64, 65]),
    (128, 16, 28, 4, [512, 1, 300, 8192 // 8]),
    (128, 256, 16, 8, [1, 255, 256, 257, 511, 512, 513, 4096]),
    (128, 32, 7, 1, [129, 33, 2000]),
    (128, 16, 12, 1, [100, 1, 777]),           # 12 heads per KV head (MFMA kernel)
    (64, 64, 16, 1, [5, 300, 1024]),           # 16 heads per KV head: one MFMA workgroup
    (128, 16, 20, 1, [700, 1, 257]),           # 20 heads: two MFMA sub-groups of 10
    (64, 32, 32, 1, [64, 1000, 3]),            # 32 heads: two MFMA sub-groups of 16
    (128, 64, 3, 1, [1, 64, 65, 1000]),        # 3 heads: the smallest MFMA group
    (128, 256, 16, 8, [3000]),                 # one sequence: its first split, then 11 more
    (128, 512, 3, 3, [1500, 2]),
    (128, 1024, 2, 2, [3000, 1025]),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"D{c[0]}_bs{c[1]}_h{c[2]}-{c[3]}" for c in SMALL])
def test_decode_small_cases(case):
    dev = device()
    D, BS, Hq, Hkv, ctx = case
    c = decode_case(1234 + D + BS + Hq, ctx, Hq, Hkv, D, BS, nb_factor=1.4)
    say(f"[decode-small] D={D} BS={BS} Hq={Hq} Hkv={Hkv} ctx={ctx}")
    d = DecodeOnDevice(c, dev)
    d.store()
    out32 = as_f64(d.decode(torch.float32))
    out16 = as_f64(d.decode(torch.bfloat16))
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    assert np.abs(out32 - ref).max() <= ATOL
    assert np.abs(out16 - ref).max() <= ATOL
    assert np.array_equal(bits(d.k_cache), kc) and np.array_equal(bits(d.v_cache), vc)
    for i, n in enumerate(ctx):
        if n == 0:
            assert np.all(out32[i] == 0) and np.all(out16[i] == 0)
        if n == 1:  # one key: the output is that token's V exactly
            G = Hq // Hkv
            for h in range(Hq):
                assert np.array_equal(out32[i, h], oracle.bf16_to_f64(c.v_new[i, h // G]))


def test_decode_block_permutation_bit_identical():
    dev = device()
    c = decode_case(77, [300, 1, 513, 40, 1024], 8, 2, 128, 16, nb_factor=1.5)
    d = DecodeOnDevice(c, dev)
    d.store()
    a = d.decode(torch.float32)
    perm = np.random.default_rng(78).permutation(c.num_blocks)
    kc, vc = bits(d.k_cache), bits(d.v_cache)
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm] = kc
    vp[perm] = vc
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1)
    b = d.decode(torch.float32, tables=i32(bt, dev), k_cache=bf16(kp, dev), v_cache=bf16(vp, dev))
    assert torch.equal(a, b)


def test_decode_deterministic_and_workspace_reuse():
    """Repeated calls are bit-identical, also after a different-shaped call reused the workspace."""
    dev = device()
    c1 = decode_case(80, [4000, 17, 2600, 900, 1], 16, 8, 128, 256, num_blocks=64,
                     max_blocks_per_seq=16)
    c2 = decode_case(81, [100, 3000], 16, 8, 128, 256, num_blocks=32, max_blocks_per_seq=16)
    d1, d2 = DecodeOnDevice(c1, dev), DecodeOnDevice(c2, dev)
    d1.store()
    d2.store()
    nbytes = max(pa.decode_workspace_bytes(5, 16, 8, 128, 256, 16),
                 pa.decode_workspace_bytes(2, 16, 8, 128, 256, 16))
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=dev)  # needs no initialisation
    a = d1.decode(torch.float32, workspace=ws)
    b = d2.decode(torch.float32, workspace=ws)
    a2 = d1.decode(torch.float32, workspace=ws)
    assert torch.equal(a, a2)
    kc, vc = oracle.kvcache_store(c2.k_new, c2.v_new, c2.slot_mapping, c2.k_cache, c2.v_cache)
    ref = oracle.paged_decode(c2.q, kc, vc, c2.block_tables, c2.context_lens, np.float32(c2.scale))
    assert np.abs(as_f64(b) - ref).max() <= ATOL


def test_decode_reads_new_token_from_cache():
    """Decode after the store equals decode over a pool where that token was placed by the oracle."""
    dev = device()
    c = decode_case(82, [33, 260, 7], 4, 2, 64, 16, nb_factor=1.5)
    d = DecodeOnDevice(c, dev)
    d.store()
    a = d.decode(torch.float32)
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    b = d.decode(torch.float32, k_cache=bf16(kc, dev), v_cache=bf16(vc, dev))
    assert torch.equal(a, b)


def test_decode_workspace_shared_by_different_shapes():
    """A workspace used by one shape, then by a shape with more (sequence, head group) pairs."""
    dev = device()
    a = decode_case(83, [2000, 1500, 3000, 700], 28, 4, 128, 16, nb_factor=1.3)
    b = decode_case(84, list(range(300, 300 + 64 * 9, 9)), 16, 8, 128, 256, nb_factor=1.3)
    nbytes = max(pa.decode_workspace_bytes(a.batch, 28, 4, 128, 16, a.max_blocks_per_seq),
                 pa.decode_workspace_bytes(b.batch, 16, 8, 128, 256, b.max_blocks_per_seq))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    for c in (a, b, a, b):
        d = DecodeOnDevice(c, dev)
        d.store()
        got = as_f64(d.decode(torch.float32, workspace=ws))
        kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
        ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
        assert np.abs(got - ref).max() <= ATOL


def check_append(c, dev, label, ref=None):
    """Fused store + decode: caches as after the store (bit-exact), outputs of every sequence
    within ATOL (``ref``: the oracle's outputs when already computed)."""
    d = DecodeOnDevice(c, dev)
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        # the second call appends the same rows again: same slots, same values
        out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=dt, device=dev)
        pa.paged_decode_append(d.q, d.k_new, d.v_new, d.slots, d.k_cache, d.v_cache, d.tables,
                               d.ctx, c.scale, out)
        outs[dt] = as_f64(out)
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    assert np.array_equal(bits(d.k_cache), kc) and np.array_equal(bits(d.v_cache), vc)
    if ref is None:
        ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens,
                                  np.float32(c.scale))
    e32 = np.abs(outs[torch.float32] - ref).max()
    e16 = np.abs(outs[torch.bfloat16] - ref).max()
    say(f"[append] {label}: max|err| fp32 {e32:.3e} bf16 {e16:.3e} over all {c.batch} seqs")
    assert e32 <= ATOL and e16 <= ATOL
    return outs[torch.float32]


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_decode_append_workload(cfg_id):
    dev = device()
    c = workload(cfg_id)
    check_append(c, dev, f"workload {cfg_id}", oracle_decode(cfg_id))


APPEND_SMALL = SMALL + [(64, 16, 4, 2, [512, 513, 1025, 1, 0])]


@pytest.mark.parametrize("case", APPEND_SMALL,
                         ids=[f"D{c[0]}_bs{c[1]}_h{c[2]}-{c[3]}" for c in APPEND_SMALL])
def test_decode_append_small_cases(case):
    dev = device()
    D, BS, Hq, Hkv, ctx = case
    c = decode_case(2468 + D + BS + Hq, ctx, Hq, Hkv, D, BS, nb_factor=1.4)
    out32 = check_append(c, dev, f"D{D} bs{BS} h{Hq}/{Hkv}")
    G = Hq // Hkv
    for i, n in enumerate(ctx):
        if n == 0:
            assert np.all(out32[i] == 0)
        if n == 1:  # the only key is the appended token: out = v_new exactly
            for h in range(Hq):
                assert np.array_equal(out32[i, h], oracle.bf16_to_f64(c.v_new[i, h // G]))


def _long_split_case(seed, D, BS, B=128):
    """B x 16/8 heads, blocks holding a whole split: a grid big enough for splits of twice the
    length; contexts at every split-length boundary of both kinds, the rest drawn uniformly."""
    S = 256 if D == 128 else 512  # short split length
    edges = [1, 2, S - 1, S, S + 1, 8 * S - 1, 8 * S, 8 * S + 1, 9 * S, 9 * S + 1, 10 * S - 1,
             16 * S - 1, 16 * S, 0, 2 * S, 2 * S + 1]
    rng = np.random.default_rng(seed)
    ctx = edges + [int(x) for x in rng.integers(1, 16 * S, B - len(edges), endpoint=True)]
    return decode_case(seed, ctx, 16, 8, D, BS, nb_factor=1.2, max_blocks_per_seq=16 * S // BS)


@pytest.mark.parametrize("D,BS", [(128, 256), (128, 1024), (64, 512)])
def test_decode_long_splits(D, BS):
    """Contexts longer than the grid's short-split slots take splits of twice the length (over
    two blocks or inside one): every sequence (both split kinds and every boundary) against the
    oracle, plain and fused store."""
    dev = device()
    c = _long_split_case(4321 + D + BS, D, BS)
    B = c.batch  # 128 x 8 head groups x 8 long-split slots = 8192 workgroups: long splits on,
    # so the plan at 128 needs less than 127 sequences with short splits (the size is the most)
    ws = [pa.decode_workspace_bytes(b, 16, 8, D, BS, c.max_blocks_per_seq) for b in (126, 127, B)]
    assert ws[0] < ws[1] == ws[2]
    say(f"[decode-long] D={D} BS={BS} B={B} ctx max {int(c.context_lens.max())}")
    d = DecodeOnDevice(c, dev)
    d.store()
    out32 = as_f64(d.decode(torch.float32))
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    err = np.abs(out32 - ref).max()
    say(f"[decode-long] D={D} BS={BS}: max|err| {err:.3e}")
    assert err <= ATOL
    check_append(c, dev, f"long splits D{D} BS{BS}")


def _mfma_long_case(seed, D, BS, B=128):
    """B x 28/4 heads (7 query heads per KV head: the MFMA kernel) with 8,192-token tables: at
    128 sequences the grid with 2,048-token splits still has 2,048 workgroups, so the long
    split length is taken; contexts at both split lengths' boundaries, the rest uniform."""
    S, L = 256, 2048
    edges = [1, 2, S - 1, S, S + 1, L - 1, L, L + 1, 2 * L - 1, 2 * L, 2 * L + 1, 3 * L + S,
             4 * L - 1, 4 * L, 0, 17]
    rng = np.random.default_rng(seed)
    ctx = edges + [int(x) for x in rng.integers(1, 4 * L, B - len(edges), endpoint=True)]
    return decode_case(seed, ctx, 28, 4, D, BS, nb_factor=1.1, max_blocks_per_seq=4 * L // BS)


@pytest.mark.parametrize("D,BS", [(128, 16), (64, 1), (128, 1024)])
def test_decode_mfma_long_splits(D, BS):
    """The MFMA kernel's 2,048-token splits (one chunk of loads in flight per wave, the block
    ids of a split staged in LDS — 2,048 of them at block size 1 — or a split over two
    blocks): every sequence against the oracle, plain and fused store, and
    the same outputs bit for bit from a NaN-filled workspace (every partial the merge reads was
    written by this call)."""
    dev = device()
    c = _mfma_long_case(5151 + D + BS, D, BS)
    B = c.batch
    # the switch to long splits happens at 128 sequences: the size is the most a smaller
    # batch with short splits needs
    ws = [pa.decode_workspace_bytes(b, 28, 4, D, BS, c.max_blocks_per_seq) for b in (126, 127, B)]
    assert ws[0] < ws[1] == ws[2]
    say(f"[decode-mfma-long] D={D} BS={BS} B={B} ctx max {int(c.context_lens.max())}")
    d = DecodeOnDevice(c, dev)
    d.store()
    out32 = as_f64(d.decode(torch.float32))
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    err = np.abs(out32 - ref).max()
    say(f"[decode-mfma-long] D={D} BS={BS}: max|err| {err:.3e}")
    assert err <= ATOL
    assert np.all(out32[list(c.context_lens).index(0)] == 0)
    nan_ws = torch.full((ws[2],), 0xFF, dtype=torch.uint8, device=dev)
    assert np.array_equal(as_f64(d.decode(torch.float32, workspace=nan_ws)), out32)
    check_append(c, dev, f"mfma long splits D{D} BS{BS}", ref=ref)


def test_decode_mfma_long_splits_split_major():
    """300 sequences (past the compacted list) with 2,048-token MFMA splits: the grid's slots
    go split-major from the last slot down; every sequence against the oracle, plain and fused
    store, and the same outputs from a NaN-filled workspace."""
    dev = device()
    c = _mfma_long_case(5353, 128, 16, B=300)
    say(f"[decode-mfma-long] split-major B={c.batch} ctx max {int(c.context_lens.max())}")
    d = DecodeOnDevice(c, dev)
    d.store()
    out32 = as_f64(d.decode(torch.float32))
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    err = np.abs(out32 - ref).max()
    say(f"[decode-mfma-long] split-major: max|err| {err:.3e}")
    assert err <= ATOL
    nan_ws = torch.full((pa.decode_workspace_bytes(c.batch, 28, 4, 128, 16, c.max_blocks_per_seq),),
                        0xFF, dtype=torch.uint8, device=dev)
    assert np.array_equal(as_f64(d.decode(torch.float32, workspace=nan_ws)), out32)
    check_append(c, dev, "mfma long splits, split-major", ref=ref)


MAX_CASES = [(128, 2), (128, 7), (64, 2), (64, 7)]  # VALU (2 heads per KV head) and MFMA (7)


@pytest.mark.parametrize("D,Hq", MAX_CASES, ids=[f"D{d}_h{h}-1" for d, h in MAX_CASES])
def test_decode_max_context(D, Hq):
    """The longest context one decode call takes (256 short splits: 65,536 tokens, or 131,072 on
    the head_dim-64 VALU kernel, whose splits are 512 tokens) with a table exactly that wide,
    next to one-token and short contexts; store then decode, and the fused call."""
    dev = device()
    S = 512 if (D == 64 and Hq == 2) else 256
    maxc, BS = 256 * S, 256
    ctx = [maxc, 1, maxc - 1, 300]
    c = decode_case(9100 + D + Hq, ctx, Hq, 1, D, BS, nb_factor=1.05, max_blocks_per_seq=maxc // BS)
    assert pa.decode_workspace_bytes(c.batch, Hq, 1, D, BS, c.max_blocks_per_seq) > 0
    say(f"[decode-max] D={D} h={Hq}/1 ctx={ctx}")
    d = DecodeOnDevice(c, dev)
    d.store()
    out32 = as_f64(d.decode(torch.float32))
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    err = np.abs(out32 - ref).max()
    say(f"[decode-max] D={D} h={Hq}/1: max|err| {err:.3e}")
    assert err <= ATOL
    check_append(c, dev, f"max context D{D} h{Hq}/1")


def test_decode_mfma_long_splits_max_context():
    """The longest context on the MFMA kernel's 2,048-token splits: 8 sequences x 56/8 heads
    (7 per KV head) with 65,536-token tables is the smallest batch whose grid takes them (32
    splits per context, merged past the merge's first 16-split batch), next to one-token,
    empty and boundary contexts; store then decode, and the fused call."""
    dev = device()
    maxc, BS = 65536, 256
    ctx = [maxc, 1, maxc - 1, 300, 2048, 2049, 0, 4097]
    c = decode_case(9177, ctx, 56, 8, 128, BS, nb_factor=1.05, max_blocks_per_seq=maxc // BS)
    ws = [pa.decode_workspace_bytes(b, 56, 8, 128, BS, maxc // BS) for b in (6, 7, 8)]
    assert ws[0] < ws[1] == ws[2]  # long splits from 8 sequences on
    say(f"[decode-mfma-long-max] 56/8 heads ctx={ctx}")
    d = DecodeOnDevice(c, dev)
    d.store()
    out32 = as_f64(d.decode(torch.float32))
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    err = np.abs(out32 - ref).max()
    say(f"[decode-mfma-long-max] max|err| {err:.3e}")
    assert err <= ATOL
    assert np.all(out32[6] == 0)
    check_append(c, dev, "mfma long splits, max context", ref=ref)


COMPACT_CASES = [(4, 2, 256), (14, 2, 16)]  # (Hq, Hkv, block size): VALU kernel, MFMA kernel


@pytest.mark.parametrize("Hq,Hkv,BS", COMPACT_CASES, ids=[f"h{a}-{b}_bs{c}" for a, b, c in COMPACT_CASES])
def test_decode_compact_list_matches_index_order(Hq, Hkv, BS):
    """Batches of up to 256 sequences take their splits from a compacted list, larger batches
    split-major from the last split slot down: 256 sequences, and the same 256 plus one padded
    row (257, split-major), give bit-identical outputs, plain and fused; the padded row is
    zero; both match the oracle."""
    dev = device()
    rng = np.random.default_rng(5150 + Hq)
    ctx = [0, 1, 255, 256, 257, 2048] + [int(x) for x in rng.integers(0, 2048, 250, endpoint=True)]
    c = decode_case(5150 + Hq, ctx, Hq, Hkv, 128, BS, nb_factor=1.2,
                    max_blocks_per_seq=2048 // BS)
    d = DecodeOnDevice(c, dev)
    say(f"[decode-compact] h={Hq}/{Hkv} bs={BS} B=256 vs 257")
    D, MBS = c.head_dim, c.max_blocks_per_seq

    def grow(t, fill):
        pad = torch.full((1,) + tuple(t.shape[1:]), fill, dtype=t.dtype, device=dev)
        return torch.cat([t, pad]).contiguous()

    q2, tables2, ctx2 = grow(d.q, 0), grow(d.tables, -1), grow(d.ctx, 0)
    kn2, vn2, slots2 = grow(d.k_new, 0), grow(d.v_new, 0), grow(d.slots, -1)
    d.store()
    outs = {}
    for B, (q, tables, lens) in ((256, (d.q, d.tables, d.ctx)), (257, (q2, tables2, ctx2))):
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        pa.paged_decode(q, d.k_cache, d.v_cache, tables, lens, c.scale, out)
        outs[B] = out
    assert torch.equal(outs[256], outs[257][:256])
    assert torch.count_nonzero(outs[257][256]).item() == 0
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    err = np.abs(as_f64(outs[256]) - ref).max()
    say(f"[decode-compact] h={Hq}/{Hkv} bs={BS}: max|err| {err:.3e}")
    assert err <= ATOL
    # the fused call, on caches that already hold the new rows (same slots, same values)
    fused = {}
    for B, args in ((256, (d.q, d.k_new, d.v_new, d.slots, d.tables, d.ctx)),
                    (257, (q2, kn2, vn2, slots2, tables2, ctx2))):
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        qq, kk, vv, ss, tt, ll = args
        pa.paged_decode_append(qq, kk, vv, ss, d.k_cache, d.v_cache, tt, ll, c.scale, out)
        fused[B] = out
    assert torch.equal(fused[256], fused[257][:256])
    assert np.abs(as_f64(fused[256]) - ref).max() <= ATOL


REUSE_SHAPES = [  # (Hq, Hkv, D, BS, MBS, batch): VALU short / long splits, MFMA
    (16, 8, 128, 256, 16, 64), (16, 8, 128, 256, 16, 128), (28, 4, 128, 16, 128, 40),
    (4, 2, 64, 16, 64, 33)]


def test_decode_workspace_reuse_matches_fresh_workspace():
    """The split partials go to the workspace and a second kernel merges them.  One workspace
    that starts as garbage and is reused by calls of different shapes and data, back to back on
    the stream, gives bit-identical outputs to calls on freshly zeroed workspaces (no stale
    partial is ever read)."""
    dev = device()
    rng = np.random.default_rng(4242)
    nbytes = max(pa.decode_workspace_bytes(B, Hq, Hkv, D, BS, MBS)
                 for Hq, Hkv, D, BS, MBS, B in REUSE_SHAPES)
    shared = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=dev)
    runs = []
    for it in range(12):
        Hq, Hkv, D, BS, MBS, B = REUSE_SHAPES[it % len(REUSE_SHAPES)]
        ctx = rng.integers(0, MBS * BS, size=B, endpoint=True)
        c = decode_case(7000 + it, ctx, Hq, Hkv, D, BS, nb_factor=1.2, max_blocks_per_seq=MBS)
        d = DecodeOnDevice(c, dev)
        d.store()
        runs.append((c, d, d.decode(torch.float32, workspace=shared)))  # no sync between calls
    torch.cuda.synchronize()
    say(f"[decode-reuse] {len(runs)} calls on one workspace of {nbytes} bytes")
    for c, d, got in runs:
        fresh = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        assert torch.equal(got, d.decode(torch.float32, workspace=fresh))
    c, d, got = runs[2]
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    assert np.abs(as_f64(got) - ref).max() <= ATOL
