"""Pins of the CPU oracle: checks against facts fixed outside the oracle itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees
with a closed form, a brute-force or library computation, an invariant, or a
worked example printed on the pages.  ``test_oracle.py`` runs them as tests;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle and
checks that some pin catches each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from workloads import (BF16_NAN, bf16_bits_from_f32, config, cu_seqlens_from_lens, decode_case,
                       prefill_case, slot_for_position)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SCALE64 = np.float32(0.125)  # 1/sqrt(64), exact


def _bits(values) -> np.ndarray:
    return bf16_bits_from_f32(np.asarray(values, dtype=np.float32))


def _pool_from_logical(logical, table, block_size, num_blocks):
    """Page logical rows into a NaN-filled pool one token at a time (test-side construction)."""
    Hkv, D = logical.shape[1], logical.shape[2]
    pool = np.full((num_blocks, block_size, Hkv, D), BF16_NAN, dtype=np.uint16)
    for j in range(logical.shape[0]):
        pool[table[j // block_size], j % block_size] = logical[j]
    return pool


def _single_seq_decode(q, K, V, scale, block_size=16, seed=0):
    """Oracle decode of one sequence given contiguous logical K/V ([n, Hkv, D] bits)."""
    n = K.shape[0]
    nblk = -(-n // block_size)
    rng = np.random.default_rng(seed)
    table = rng.permutation(nblk + 3)[:nblk].astype(np.int32)
    kp = _pool_from_logical(K, table, block_size, nblk + 3)
    vp = _pool_from_logical(V, table, block_size, nblk + 3)
    return oracle.paged_decode(q[None], kp, vp, table[None], np.array([n], np.int32), scale)[0]


# --------------------------------------------------------------------------- format / examples

def pin_bf16_decode():
    """bfloat16 is the top half of a float32: values fixed by the format."""
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80, 0x3F81, 0x0000, 0xC2F7], np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, math.inf, 1.0 + 2.0 ** -7, 0.0, -123.5]
    got = oracle.bf16_to_f64(bits)
    assert got.tolist() == want, got


def pin_cu_seqlens_example():
    g = json.load(open(os.path.join(GOLDEN, "cu_seqlens_example.json")))
    assert cu_seqlens_from_lens(g["q_lens"]).tolist() == g["cu_seqlens_q"]


def pin_block_boundary_example():
    """The 257th token of a sequence with block size 256 goes to offset 0 of the second block."""
    g = json.load(open(os.path.join(GOLDEN, "slot_block_boundary.json")))
    bs, table = g["block_size"], g["block_table"]
    pos = g["new_token_position"]
    assert (g["tokens_before"] % bs == 0) and ((g["tokens_before"] + 1) % bs == 1)
    slot = table[-1] * bs + g["last_block_num_tokens"] - 1
    assert slot == g["expected_slot"] == slot_for_position(table, pos, bs)
    rng = np.random.default_rng(3)
    Hkv, D, NB = 1, 64, 6
    pool_k = np.full((NB, bs, Hkv, D), BF16_NAN, np.uint16)
    first = _bits(rng.standard_normal((bs, Hkv, D)))
    pool_k[g["full_block_of_first_256"]] = first
    new_k = _bits(rng.standard_normal((1, Hkv, D)))
    kc, _ = oracle.kvcache_store(new_k, new_k, np.array([slot], np.int32), pool_k, pool_k.copy())
    assert np.array_equal(kc[g["expected_block"], g["expected_offset"]], new_k[0])
    rows = oracle.unpage(kc, np.array(table, np.int32), pos + 1)
    assert np.array_equal(rows[:bs], first)
    assert np.array_equal(rows[pos], new_k[0])


# --------------------------------------------------------------------------- store and un-page

def pin_store_writes_exactly_mapped_slots():
    rng = np.random.default_rng(5)
    NB, BS, Hkv, D, T = 9, 8, 2, 64, 20
    base = rng.integers(0, 1 << 16, size=(NB, BS, Hkv, D), dtype=np.uint16)
    k = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int32)
    slots[[3, 11]] = -1
    kc, vc = oracle.kvcache_store(k, v, slots, base, base.copy())
    where = {int(s): t for t, s in enumerate(slots) if s >= 0}
    for b in range(NB):
        for o in range(BS):
            t = where.get(b * BS + o)
            exp_k = base[b, o] if t is None else k[t]
            exp_v = base[b, o] if t is None else v[t]
            assert np.array_equal(kc[b, o], exp_k) and np.array_equal(vc[b, o], exp_v), (b, o)


def pin_unpage_round_trip():
    """Paging token by token, then un-paging, gives the logical rows back bit for bit."""
    rng = np.random.default_rng(6)
    for BS, n in ((16, 37), (8, 8), (4, 1), (32, 95)):
        nblk = -(-n // BS)
        table = rng.permutation(nblk + 5)[:nblk]
        logical = rng.integers(0, 1 << 16, size=(n, 2, 64), dtype=np.uint16)
        pool = _pool_from_logical(logical, table, BS, nblk + 5)
        assert np.array_equal(oracle.unpage(pool, table, n), logical)


def pin_generator_pages_what_oracle_unpages():
    """The workload generator's pool holds each sequence's logical rows (also shared prefixes)."""
    c = config(1, keep_logical=True)
    for i in range(c.batch):
        n = int(c.context_lens[i]) - 1
        assert np.array_equal(oracle.unpage(c.k_cache, c.block_tables[i], n), c.logical_k[i])
        assert np.array_equal(oracle.unpage(c.v_cache, c.block_tables[i], n), c.logical_v[i])
    s = decode_case(4, [40, 35, 50, 9], 2, 1, 64, 8, nb_factor=1.5, shared_groups=[[0, 2]],
                    shared_blocks=[4], keep_logical=True)
    assert s.block_tables[0, :4].tolist() == s.block_tables[2, :4].tolist()
    for i in range(s.batch):
        n = int(s.context_lens[i]) - 1
        assert np.array_equal(oracle.unpage(s.k_cache, s.block_tables[i], n), s.logical_k[i])


# --------------------------------------------------------------------------- attention values

def _brute_force(q, K, V, scale):
    """Softmax attention with Python floats and math.exp, no paging, no NumPy."""
    qf = [float(x) for x in q]
    scores = [sum(a * b for a, b in zip(qf, row)) * float(scale) for row in K]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    tot = sum(w)
    return [sum(w[j] * V[j][d] for j in range(len(V))) / tot for d in range(len(V[0]))]


def pin_decode_matches_brute_force():
    rng = np.random.default_rng(7)
    for ctx, Hq, Hkv in (([1, 9, 23], 2, 1), ([31, 5], 4, 2), ([17], 4, 1)):
        c = decode_case(int(rng.integers(1 << 30)), ctx, Hq, Hkv, 64, 8, nb_factor=2.0,
                        keep_logical=True)
        kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
        out = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, SCALE64)
        G = Hq // Hkv
        for i in range(c.batch):
            K = np.concatenate([c.logical_k[i], c.k_new[i:i + 1]])
            V = np.concatenate([c.logical_v[i], c.v_new[i:i + 1]])
            for h in range(Hq):
                g = h // G
                Kg = oracle.bf16_to_f64(K[:, g]).tolist()
                Vg = oracle.bf16_to_f64(V[:, g]).tolist()
                ref = _brute_force(oracle.bf16_to_f64(c.q[i, h]), Kg, Vg, SCALE64)
                assert np.max(np.abs(out[i, h] - np.array(ref))) < 1e-12, (i, h)


def pin_decode_matches_torch_sdpa():
    """torch's CPU scaled_dot_product_attention (float64) on the un-paged K/V."""
    import torch.nn.functional as F
    rng = np.random.default_rng(8)
    for D, BS, Hq, Hkv, ctx in ((128, 16, 8, 8, [300, 1, 129]), (128, 32, 14, 2, [77, 250]),
                                (64, 8, 8, 1, [64, 65, 3])):
        c = decode_case(int(rng.integers(1 << 30)), ctx, Hq, Hkv, D, BS, nb_factor=1.3,
                        keep_logical=True)
        kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
        scale = np.float32(1 / math.sqrt(D))
        out = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, scale)
        for i in range(c.batch):
            K = oracle.bf16_to_f64(np.concatenate([c.logical_k[i], c.k_new[i:i + 1]]))
            V = oracle.bf16_to_f64(np.concatenate([c.logical_v[i], c.v_new[i:i + 1]]))
            qt = torch.from_numpy(oracle.bf16_to_f64(c.q[i]))[:, None, :]          # [Hq, 1, D]
            Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)  # [Hq, n, D]
            Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
            ref = F.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous(),
                                                 scale=float(scale))[:, 0, :].numpy()
            assert np.max(np.abs(out[i] - ref)) < 1e-10, i


def pin_one_token_context_returns_v():
    c = decode_case(9, [1, 1, 1], 4, 2, 128, 16, nb_factor=2.0)
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    out = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(0.0883883))
    for i in range(3):
        for h in range(4):
            assert np.array_equal(out[i, h], oracle.bf16_to_f64(c.v_new[i, h // 2]))


def pin_constant_values_and_uniform_keys():
    rng = np.random.default_rng(10)
    n, D = 45, 64
    q = _bits(rng.standard_normal((1, D)))
    K = _bits(rng.standard_normal((n, 1, D)))
    V = np.broadcast_to(_bits(rng.standard_normal(D)), (n, 1, D)).copy()
    out = _single_seq_decode(q, K, V, SCALE64)
    assert np.max(np.abs(out[0] - oracle.bf16_to_f64(V[0, 0]))) < 1e-14
    K_same = np.broadcast_to(K[0], (n, 1, D)).copy()
    V_rand = _bits(rng.standard_normal((n, 1, D)))
    out = _single_seq_decode(q, K_same, V_rand, SCALE64)
    assert np.max(np.abs(out[0] - oracle.bf16_to_f64(V_rand[:, 0]).mean(axis=0))) < 1e-12
    out = _single_seq_decode(np.zeros_like(q), K, V_rand, SCALE64)
    assert np.max(np.abs(out[0] - oracle.bf16_to_f64(V_rand[:, 0]).mean(axis=0))) < 1e-12


def pin_two_key_closed_form():
    """Two keys with dot products 2 and 6, scale 1/8: weights are sigmoid(-1/2) and sigmoid(1/2)."""
    D = 64
    q = np.zeros((1, D), np.float32); q[0, 0] = 2.0
    K = np.zeros((2, 1, D), np.float32); K[0, 0, 0] = 1.0; K[1, 0, 0] = 3.0
    V = np.zeros((2, 1, D), np.float32); V[0, 0, :] = 1.0; V[1, 0, :] = -1.0; V[1, 0, 5] = 4.0
    out = _single_seq_decode(_bits(q), _bits(K), _bits(V), SCALE64)[0]
    w1 = 1.0 / (1.0 + math.exp(-0.5))
    want = (1 - w1) * 1.0 + w1 * (-1.0)
    assert abs(out[0] - want) < 1e-14 and abs(out[63] - want) < 1e-14
    assert abs(out[5] - ((1 - w1) * 1.0 + w1 * 4.0)) < 1e-14


def pin_scale_multiplies_dot_product():
    """scale 1/8 on q equals scale 1 on q/8 (q/8 is exact in bfloat16)."""
    rng = np.random.default_rng(11)
    n, D = 30, 64
    qf = rng.standard_normal((1, D)).astype(np.float32)
    q = _bits(qf)
    q8 = _bits(oracle.bf16_to_f64(q).astype(np.float32) / 8)
    K = _bits(rng.standard_normal((n, 1, D)))
    V = _bits(rng.standard_normal((n, 1, D)))
    a = _single_seq_decode(q, K, V, SCALE64)
    b = _single_seq_decode(q8, K, V, np.float32(1.0))
    assert np.max(np.abs(a - b)) < 1e-14


def pin_gqa_head_mapping():
    """KV head g holds V == g + 1 everywhere, so query head h must return h // G + 1."""
    Hq, Hkv, D, BS = 8, 4, 64, 8
    c = decode_case(13, [20, 9], Hq, Hkv, D, BS, nb_factor=2.0)
    vc = c.v_cache.copy()
    v_new = c.v_new.copy()
    for g in range(Hkv):
        val = _bits(np.float32(g + 1))
        vc[:, :, g, :] = np.where(c.v_cache[:, :, g, :] == BF16_NAN, BF16_NAN, val)
        v_new[:, g, :] = val
    kc, vc = oracle.kvcache_store(c.k_new, v_new, c.slot_mapping, c.k_cache, vc)
    out = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, SCALE64)
    for h in range(Hq):
        assert np.max(np.abs(out[:, h] - (h // (Hq // Hkv) + 1))) < 1e-14, h


def pin_gqa_equals_expanded_heads():
    """Repeating each KV head G times and running with G = 1 gives the same output."""
    Hq, Hkv = 6, 2
    c = decode_case(14, [33, 7, 18], Hq, Hkv, 64, 8, nb_factor=1.5)
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    a = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, SCALE64)
    G = Hq // Hkv
    b = oracle.paged_decode(c.q, np.repeat(kc, G, axis=2), np.repeat(vc, G, axis=2),
                            c.block_tables, c.context_lens, SCALE64)
    assert np.array_equal(a, b)


def pin_block_permutation_invariance():
    c = decode_case(15, [50, 17, 64, 3], 4, 2, 64, 16, nb_factor=1.7)
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    a = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, SCALE64)
    perm = np.random.default_rng(16).permutation(c.num_blocks)
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm] = kc
    vp[perm] = vc
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    b = oracle.paged_decode(c.q, kp, vp, bt, c.context_lens, SCALE64)
    assert np.array_equal(a, b)


def pin_padded_row_is_zero_and_unused_slots_unread():
    c = decode_case(17, [0, 20, 0, 5], 2, 1, 64, 8, nb_factor=1.5)
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    out = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, SCALE64)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isfinite(out))  # the pool's unused slots are NaN


# --------------------------------------------------------------------------- prefill

def _prefill_inputs(seed, P, n, Hq=4, Hkv=2, D=64, BS=8):
    return prefill_case(seed, P, n, Hq, Hkv, D, BS, keep_logical=True)


def pin_prefill_rows_equal_decode_steps():
    """Chunk row t equals a decode of that token over the first P + t + 1 tokens."""
    p = _prefill_inputs(18, [0, 13, 24], [6, 9, 1])
    out = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, SCALE64)
    kc, vc = oracle.kvcache_store(p.k_new, p.v_new, p.slot_mapping, p.k_cache, p.v_cache)
    for i in range(p.batch):
        for t in range(int(p.q_lens[i])):
            row = int(p.cu_seqlens_q[i]) + t
            ctx = np.array([int(p.prefix_lens[i]) + t + 1], np.int32)
            dec = oracle.paged_decode(p.q[row:row + 1], kc, vc, p.block_tables[i:i + 1], ctx,
                                      SCALE64)
            assert np.max(np.abs(out[row] - dec[0])) < 1e-12, (i, t)


def pin_prefill_first_token_without_prefix_is_its_v():
    p = _prefill_inputs(19, [0, 0], [3, 5])
    out = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, SCALE64)
    for i in range(2):
        row = int(p.cu_seqlens_q[i])
        for h in range(4):
            assert np.array_equal(out[row, h], oracle.bf16_to_f64(p.v_new[row, h // 2]))


def pin_prefill_matches_torch_sdpa_with_mask():
    import torch.nn.functional as F
    p = _prefill_inputs(20, [11, 0, 40], [7, 12, 16], Hq=6, Hkv=3, D=64, BS=16)
    out = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, SCALE64)
    for i in range(p.batch):
        a, b = int(p.cu_seqlens_q[i]), int(p.cu_seqlens_q[i + 1])
        P, n = int(p.prefix_lens[i]), b - a
        K = oracle.bf16_to_f64(np.concatenate([p.logical_k[i], p.k_new[a:b]]))
        V = oracle.bf16_to_f64(np.concatenate([p.logical_v[i], p.v_new[a:b]]))
        mask = torch.ones(n, P + n, dtype=torch.bool).tril(diagonal=P)  # bottom-right aligned
        qt = torch.from_numpy(oracle.bf16_to_f64(p.q[a:b])).permute(1, 0, 2)
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(2, 0).contiguous()
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(2, 0).contiguous()
        ref = F.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=0.125)
        assert np.max(np.abs(out[a:b] - ref.permute(1, 0, 2).numpy())) < 1e-10, i


def pin_prefill_is_causal():
    """Changing the K/V of later chunk tokens leaves earlier rows bit-identical."""
    p = _prefill_inputs(21, [9], [10])
    out = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, SCALE64)
    k2, v2 = p.k_new.copy(), p.v_new.copy()
    k2[6:] ^= 0x1234
    v2[6:] ^= 0x0F0F
    out2 = oracle.paged_prefill(p.q, k2, v2, p.cu_seqlens_q, p.k_cache, p.v_cache,
                                p.block_tables, p.context_lens, SCALE64)
    assert np.array_equal(out[:6], out2[:6])
    assert not np.array_equal(out[6:], out2[6:])




# --------------------------------------------------------------------------- FP8 KV cache

def pin_e4m3_known_codes():
    """Values fixed by the OCP FP8 E4M3 format."""
    from oracle import e4m3_decode
    want = {0x38: 1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9,
            0xBC: -1.5, 0x40: 2.0, 0x3F: 1.875, 0x00: 0.0, 0x5A: 20.0}
    for code, val in want.items():
        assert e4m3_decode([code])[0] == val, hex(code)
    assert np.isnan(e4m3_decode([0x7F])[0]) and np.isnan(e4m3_decode([0xFF])[0])
    assert np.signbit(e4m3_decode([0x80])[0]) and e4m3_decode([0x80])[0] == 0.0


def pin_e4m3_round_trip():
    from oracle import e4m3_decode, e4m3_encode
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def pin_e4m3_matches_torch_in_range():
    """torch's float8_e4m3fn cast (round to nearest even) on in-range values, midpoints included."""
    from oracle import e4m3_decode, e4m3_encode
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = 0.5 * (vals[:-1] + vals[1:])
    rng = np.random.default_rng(30)
    x = np.concatenate([mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 0.01]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), ref)


def pin_e4m3_saturates():
    from oracle import e4m3_encode
    got = e4m3_encode(np.array([448.0, 463.9, 464.0, 480.0, 1e6, np.inf, -1e9, -np.inf]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert (e4m3_encode(np.array([np.nan]))[0] & 0x7F) == 0x7F


def pin_fp8_quantize_matches_torch_every_bf16():
    """Every bf16 pattern (NaNs of both signs, subnormals, signed zeros) at scales that are not
    powers of two: the code equals torch's float32 division followed by its float8_e4m3fn cast
    (round to nearest even, NaN keeps its sign).  Quotients beyond 448 are left out: torch
    turns them into NaN, where the quantizer saturates (pinned literally above)."""
    from oracle import quantize
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x32 = torch.from_numpy((bits.astype(np.uint32) << 16).view(np.float32))
    for s in (0.3, 0.017, 0.0107, 0.7, 1.0 / 64, 1.7):
        q32 = x32 / torch.tensor(s, dtype=torch.float32)
        ref = q32.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        keep = (torch.isnan(q32) | (q32.abs() <= 448.0)).numpy()
        with np.errstate(over="ignore", invalid="ignore"):
            got = quantize(bits, s)
        bad = np.nonzero((got != ref) & keep)[0]
        assert bad.size == 0, f"scale {s}: {bad.size} codes differ, first bf16 0x{bits[bad[0]]:04x}"
    # both NaN signs are among the patterns compared
    nan_codes = quantize(np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFF81], np.uint16), 0.3)
    assert nan_codes.tolist() == [0x7F, 0xFF, 0x7F, 0xFF]


def pin_fp8_quantize_power_of_two_scale():
    """Dividing by 2^k before rounding equals rounding the exponent-shifted value."""
    from oracle import e4m3_encode, quantize
    rng = np.random.default_rng(31)
    bits = _bits(rng.standard_normal(3000) * 40)
    x = oracle.bf16_to_f64(bits)
    for k in (-3, 0, 2):
        assert np.array_equal(quantize(bits, 2.0 ** k), e4m3_encode(x / 2.0 ** k))


def pin_fp8_decode_reduces_to_bf16_decode():
    """With values exactly representable in E4M3 and scales 1, FP8 decode equals the bf16 decode."""
    from oracle import paged_decode_fp8
    c = decode_case(32, [40, 7, 100], 4, 2, 64, 16, nb_factor=1.5)
    rng = np.random.default_rng(33)
    codes_k = rng.integers(0, 0x7F, size=c.k_cache.shape).astype(np.uint8) | (
        rng.integers(0, 2, size=c.k_cache.shape).astype(np.uint8) << 7)
    codes_v = rng.integers(0, 0x7F, size=c.v_cache.shape).astype(np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x38
    vals_k = oracle.e4m3_decode(codes_k).astype(np.float32)
    vals_v = oracle.e4m3_decode(codes_v).astype(np.float32)
    bits_k = (vals_k.view(np.uint32) >> 16).astype(np.uint16)  # exact: E4M3 fits in bf16
    bits_v = (vals_v.view(np.uint32) >> 16).astype(np.uint16)
    a = paged_decode_fp8(c.q, codes_k, codes_v, c.block_tables, c.context_lens, SCALE64, 1.0, 1.0)
    b = oracle.paged_decode(c.q, bits_k, bits_v, c.block_tables, c.context_lens, SCALE64)
    assert np.array_equal(a, b)
    # scales multiply K and V
    a2 = paged_decode_fp8(c.q, codes_k, codes_v, c.block_tables, c.context_lens, SCALE64, 0.5, 4.0)
    bits_k2 = ((vals_k * 0.5).view(np.uint32) >> 16).astype(np.uint16)
    bits_v2 = ((vals_v * 4.0).view(np.uint32) >> 16).astype(np.uint16)
    b2 = oracle.paged_decode(c.q, bits_k2, bits_v2, c.block_tables, c.context_lens, SCALE64)
    assert np.max(np.abs(a2 - b2)) < 1e-12


def _fp8_prefill_inputs(seed, prefix_lens, q_lens, k_scale, v_scale, Hq=4, Hkv=2, D=64, BS=16):
    """A prefill chunk with FP8 pools holding the prefix and, stored, the chunk's own tokens."""
    from oracle import kvcache_store_fp8, quantize
    p = _prefill_inputs(seed, prefix_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D, BS=BS)
    kc8, vc8 = kvcache_store_fp8(p.k_new, p.v_new, p.slot_mapping, quantize(p.k_cache, k_scale),
                                 quantize(p.v_cache, v_scale), k_scale, v_scale)
    return p, kc8, vc8


def pin_fp8_prefill_rows_equal_fp8_decode_steps():
    """Chunk row t over an FP8 cache equals an FP8 decode of that token over P + t + 1 keys."""
    from oracle import paged_decode_fp8, paged_prefill_fp8
    ks, vs = 0.013, 0.021
    p, kc8, vc8 = _fp8_prefill_inputs(35, [0, 13, 24], [6, 9, 1], ks, vs)
    out = paged_prefill_fp8(p.q, p.cu_seqlens_q, kc8, vc8, p.block_tables, p.context_lens,
                            SCALE64, ks, vs)
    for i in range(p.batch):
        for t in range(int(p.q_lens[i])):
            row = int(p.cu_seqlens_q[i]) + t
            ctx = np.array([int(p.prefix_lens[i]) + t + 1], np.int32)
            dec = paged_decode_fp8(p.q[row:row + 1], kc8, vc8, p.block_tables[i:i + 1], ctx,
                                   SCALE64, ks, vs)
            assert np.max(np.abs(out[row] - dec[0])) < 1e-12, (i, t)


def pin_fp8_prefill_reduces_to_bf16_prefill():
    """Scales 1 and values exactly representable in E4M3: FP8 prefill equals the bf16 prefill
    whose prefix and new K/V are those values (bit-exact: bf16 holds every E4M3 value)."""
    from oracle import paged_prefill_fp8
    p = _prefill_inputs(36, [5, 40], [7, 3], Hq=6, Hkv=2, D=64, BS=8)
    rng = np.random.default_rng(37)
    kc8 = rng.integers(0, 0x7F, size=p.k_cache.shape).astype(np.uint8) | (
        rng.integers(0, 2, size=p.k_cache.shape).astype(np.uint8) << 7)
    vc8 = rng.integers(0, 0x7F, size=p.v_cache.shape).astype(np.uint8)

    def bits(codes):
        return (oracle.e4m3_decode(codes).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kb, vb = bits(kc8), bits(vc8)
    slots = p.slot_mapping
    k_new = np.stack([kb[s // 8, s % 8] for s in slots])
    v_new = np.stack([vb[s // 8, s % 8] for s in slots])
    a = paged_prefill_fp8(p.q, p.cu_seqlens_q, kc8, vc8, p.block_tables, p.context_lens, SCALE64,
                          1.0, 1.0)
    b = oracle.paged_prefill(p.q, k_new, v_new, p.cu_seqlens_q, kb, vb, p.block_tables,
                             p.context_lens, SCALE64)
    assert np.array_equal(a, b)


def pin_fp8_store_writes_exactly_mapped_slots():
    from oracle import kvcache_store_fp8, quantize
    rng = np.random.default_rng(34)
    NB, BS, Hkv, D, T = 6, 8, 2, 64, 15
    base = rng.integers(0, 256, size=(NB, BS, Hkv, D), dtype=np.uint8)
    k = _bits(rng.standard_normal((T, Hkv, D)) * 3)
    v = _bits(rng.standard_normal((T, Hkv, D)))
    slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int32)
    slots[[2, 9]] = -1
    kc, vc = kvcache_store_fp8(k, v, slots, base, base.copy(), 0.03, 0.5)
    where = {int(s): t for t, s in enumerate(slots) if s >= 0}
    kq, vq = quantize(k, 0.03), quantize(v, 0.5)
    for b in range(NB):
        for o in range(BS):
            t = where.get(b * BS + o)
            assert np.array_equal(kc[b, o], base[b, o] if t is None else kq[t])
            assert np.array_equal(vc[b, o], base[b, o] if t is None else vq[t])


# --------------------------------------------------------------------------- block manager

def pin_fnv1a_published_vectors():
    """64-bit FNV-1a test vectors published with the algorithm."""
    from oracle import fnv1a64
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def pin_block_hash_bytes():
    """The chained block hash is FNV-1a of the predecessor's hash then the token ids, LE."""
    from oracle import block_hash, fnv1a64
    toks = [1, 2, 3, 70000]
    first = b"".join(t.to_bytes(4, "little") for t in toks)
    assert block_hash(toks, -1) == fnv1a64(first)
    prev = 0x0123456789ABCDEF
    assert block_hash(toks, prev) == fnv1a64(prev.to_bytes(8, "little") + first)
    assert block_hash(toks, prev, 5) == fnv1a64(prev.to_bytes(8, "little") + first) & 31
    # the same tokens under another prefix hash differently (the pages' [prefix1][1,2,3] example)
    assert block_hash([1, 2, 3], 11) != block_hash([1, 2, 3], 12)


def pin_block_manager_boundary_example():
    """The 257th token of a sequence with one full 256-token block opens a new block at offset 0
    (the pages' prepare_decode example, stored in tests/golden/slot_block_boundary.json)."""
    g = json.load(open(os.path.join(GOLDEN, "slot_block_boundary.json")))
    bs = g["block_size"]
    bm = oracle.BlockManager(8, bs)
    bm.allocate(1, list(range(g["tokens_before"])))
    assert len(bm.block_table(1)) == 1
    bm.append(1, 99)
    t = bm.block_table(1)
    assert len(t) == 2
    assert bm.decode_slot(1) == t[1] * bs + g["expected_offset"]
    # a sequence's own tokens before the boundary stay in its first block
    assert bm.prefill_slots(1)[g["tokens_before"] - 1] == t[0] * bs + bs - 1


def pin_block_manager_prefix_sharing():
    """Two prompts with the same two full blocks share their physical blocks (ref count 2) and
    the second sees 2*BS cached tokens; the partial tails are private."""
    bs = 4
    bm = oracle.BlockManager(16, bs)
    a = [5, 6, 7, 8, 9, 10, 11, 12, 1, 2]
    b = [5, 6, 7, 8, 9, 10, 11, 12, 3]
    assert bm.allocate(1, a) == 0
    assert bm.allocate(2, b) == 2 * bs
    ta, tb = bm.block_table(1), bm.block_table(2)
    assert ta[:2] == tb[:2] and ta[2] != tb[2]
    assert [bm.blocks[x].ref_count for x in ta] == [2, 2, 1]
    assert bm.prefill_slots(2) == [tb[2] * bs + 0]
    assert len(bm.free) == 16 - 4
    # a prompt that is a strict prefix shares only full blocks
    assert bm.allocate(3, a[:6]) == bs
    assert bm.block_table(3)[0] == ta[0] and bm.block_table(3)[1] not in ta


def pin_block_manager_chained_hash_blocks_false_reuse():
    """A block with the same tokens after a different first block is not reused."""
    bs = 3
    bm = oracle.BlockManager(10, bs)
    bm.allocate(1, [1, 2, 3, 7, 8, 9])
    assert bm.allocate(2, [4, 5, 6, 7, 8, 9]) == 0
    assert set(bm.block_table(1)).isdisjoint(bm.block_table(2))


def pin_block_manager_cache_survives_free():
    """Freed blocks stay findable: the same prompt again hits every full block, and the freed
    blocks come back off the free list; deallocation frees the last block first."""
    bs = 4
    bm = oracle.BlockManager(8, bs)
    toks = list(range(100, 111))  # 2 full blocks + 3 tokens
    bm.allocate(1, toks)
    t1 = bm.block_table(1)
    bm.deallocate(1)
    assert list(bm.free)[-3:] == t1[::-1]
    assert bm.allocate(2, toks) == 2 * bs
    t2 = bm.block_table(2)
    assert t2[:2] == t1[:2]
    assert all(bm.blocks[x].ref_count == 1 for x in t2)
    assert len(bm.free) == 8 - 3


def pin_block_manager_append_hashes_full_blocks():
    """Decode appends fill the last block; once full it is hashed and a new prompt with the
    same tokens hits it."""
    bs = 4
    bm = oracle.BlockManager(8, bs)
    bm.allocate(1, [1, 2])
    for t in (3, 4, 5):
        assert bm.can_append(1)
        bm.append(1, t)
    assert len(bm.block_table(1)) == 2
    assert bm.allocate(2, [1, 2, 3, 4, 9]) == bs
    assert bm.block_table(2)[0] == bm.block_table(1)[0]


def _bm_check_invariants(bm):
    n = len(bm.blocks)
    free = list(bm.free)
    assert len(set(free)) == len(free)
    assert set(free).isdisjoint(bm.used) and set(free) | bm.used == set(range(n))
    counts = {}
    for sq in bm.seqs.values():
        for x in sq.block_table:
            counts[x] = counts.get(x, 0) + 1
        bs = bm.block_size
        assert len(sq.block_table) == -(-len(sq.token_ids) // bs)
        for i, x in enumerate(sq.block_table):
            toks = sq.token_ids[i * bs:(i + 1) * bs]
            if len(toks) == bs:  # a full block holds exactly this sequence's tokens
                assert bm.blocks[x].token_ids == toks
        if sq.token_ids:
            p = len(sq.token_ids) - 1
            assert bm.decode_slot(sq.seq_id) == sq.block_table[p // bs] * bs + p % bs
    for x in range(n):
        assert bm.blocks[x].ref_count == counts.get(x, 0)
    # slots of partial (last, unfilled) blocks belong to one sequence only
    partial = [sq.block_table[-1] for sq in bm.seqs.values()
               if sq.token_ids and len(sq.token_ids) % bm.block_size]
    assert len(partial) == len(set(partial))


def pin_block_manager_random_invariants():
    """Random allocate / append / deallocate runs keep the books straight, also with a 3-bit
    hash where collisions are frequent (the token compare keeps distinct contents apart)."""
    for hash_bits, seed in ((64, 40), (3, 41), (1, 42)):
        rng = np.random.default_rng(seed)
        bm = oracle.BlockManager(40, 4, hash_bits)
        prompts = [list(rng.integers(0, 3, size=12)) for _ in range(4)]
        live = []
        for step in range(400):
            op = rng.integers(0, 3)
            if op == 0 and len(live) < 8:
                base = prompts[rng.integers(0, len(prompts))]
                toks = base[:rng.integers(1, 13)] + list(rng.integers(0, 3, size=rng.integers(0, 6)))
                if bm.can_allocate(len(toks)):
                    sid = 1000 + step
                    bm.allocate(sid, toks)
                    live.append(sid)
            elif op == 1 and live:
                sid = live[rng.integers(0, len(live))]
                if bm.can_append(sid):
                    bm.append(sid, int(rng.integers(0, 3)))
            elif op == 2 and live:
                sid = live.pop(rng.integers(0, len(live)))
                bm.deallocate(sid)
            _bm_check_invariants(bm)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
