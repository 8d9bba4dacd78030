"""Scores that climb along the context: key t of a KV head is about (A t / 256) u_h and every
query of that head is about u_h, so each later stretch of keys beats the running maximum by far
more than 2^8 (exp2 units).  The online-softmax rescale then runs chunk after chunk in every
kernel — the VALU decode's exact update, its FP8 form's stale-maximum rule, the MFMA decode's
rescale-on-growth, the prefill's 2^8 rule — and the outputs still match the oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_86_amd as pa
from gpu_util import DecodeOnDevice, as_f64, bf16, bits, device, i32, say
from workloads import bf16_bits_from_f32, decode_case, prefill_case, slot_for_position

pytestmark = pytest.mark.gpu

ATOL = 1e-2
A = 3.0  # slope of the key scale per 256 positions: ~0.19 exp2 units of score per token at D 128


def _directions(rng, Hkv, D):
    return rng.choice(np.array([-1.0, 1.0], np.float32), size=(Hkv, D))


def _key(rng, u, pos):
    """Keys of all KV heads at one position: (A pos / 256) u plus a little noise."""
    return (A * pos / 256.0) * u + 0.25 * rng.standard_normal(u.shape).astype(np.float32)


def _queries(rng, u, n, Hq):
    G = Hq // u.shape[0]
    q = np.repeat(u, G, axis=0)[None, :, :] + 0.1 * rng.standard_normal((n, Hq, u.shape[1]))
    return bf16_bits_from_f32(q.astype(np.float32))


def climbing_decode(seed, ctx, Hq, Hkv, D, BS):
    c = decode_case(seed, ctx, Hq, Hkv, D, BS, nb_factor=1.2)
    rng = np.random.default_rng(seed + 1)
    u = _directions(rng, Hkv, D)
    for i, n in enumerate(c.context_lens):
        for t in range(max(int(n) - 1, 0)):
            s = slot_for_position(c.block_tables[i], t, BS)
            c.k_cache[s // BS, s % BS] = bf16_bits_from_f32(_key(rng, u, t))
        if n > 0:
            c.k_new[i] = bf16_bits_from_f32(_key(rng, u, int(n) - 1))
    c.q[:] = _queries(rng, u, c.batch, Hq)
    return c


DECODE_CASES = [(4, 2), (28, 4)]  # VALU kernel (2 query heads per KV head), MFMA kernel (7)


@pytest.mark.parametrize("Hq,Hkv", DECODE_CASES, ids=["valu", "mfma"])
def test_decode_climbing_scores(Hq, Hkv):
    dev = device()
    c = climbing_decode(3131 + Hq, [1000, 3000, 257, 64, 1], Hq, Hkv, 128, 16)
    say(f"[rescale] decode {Hq}/{Hkv} heads ctx={list(c.context_lens)}")
    d = DecodeOnDevice(c, dev)
    out = torch.empty((c.batch, Hq, 128), dtype=torch.float32, device=dev)
    pa.paged_decode_append(d.q, d.k_new, d.v_new, d.slots, d.k_cache, d.v_cache, d.tables,
                           d.ctx, c.scale, out)
    torch.cuda.synchronize()
    kc, vc = oracle.kvcache_store(c.k_new, c.v_new, c.slot_mapping, c.k_cache, c.v_cache)
    assert np.array_equal(bits(d.k_cache), kc) and np.array_equal(bits(d.v_cache), vc)
    ref = oracle.paged_decode(c.q, kc, vc, c.block_tables, c.context_lens, np.float32(c.scale))
    err = np.abs(as_f64(out) - ref).max()
    say(f"[rescale] decode {Hq}/{Hkv}: max|err| {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("Hq,Hkv", DECODE_CASES, ids=["valu", "mfma"])
def test_decode_fp8_climbing_scores(Hq, Hkv):
    dev = device()
    c = climbing_decode(3232 + Hq, [1000, 3000, 257, 64, 1], Hq, Hkv, 128, 16)
    ks, vs = 0.08, 0.02  # the largest keys (~35) stay below 448 codes
    NB = c.k_cache.shape[0]
    kc = torch.empty((NB, 16, Hkv, 128), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    every = np.arange(NB * 16, dtype=np.int32)
    pa.kvcache_store_fp8(bf16(c.k_cache.reshape(NB * 16, Hkv, 128), dev),
                         bf16(c.v_cache.reshape(NB * 16, Hkv, 128), dev), i32(every, dev), kc, vc,
                         ks, vs)
    out = torch.empty((c.batch, Hq, 128), dtype=torch.float32, device=dev)
    pa.paged_decode_append_fp8(bf16(c.q, dev), bf16(c.k_new, dev), bf16(c.v_new, dev),
                               i32(c.slot_mapping, dev), kc, vc, i32(c.block_tables, dev),
                               i32(c.context_lens, dev), c.scale, ks, vs, out)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):
        kc8, vc8 = oracle.kvcache_store_fp8(c.k_new, c.v_new, c.slot_mapping,
                                            oracle.quantize(c.k_cache, ks),
                                            oracle.quantize(c.v_cache, vs), ks, vs)
    assert np.array_equal(kc.cpu().numpy(), kc8) and np.array_equal(vc.cpu().numpy(), vc8)
    ref = oracle.paged_decode_fp8(c.q, kc8, vc8, c.block_tables, c.context_lens,
                                  np.float32(c.scale), ks, vs)
    err = np.abs(as_f64(out) - ref).max()
    say(f"[rescale] FP8 decode {Hq}/{Hkv}: max|err| {err:.3e}")
    assert err <= ATOL


def test_prefill_climbing_scores():
    dev = device()
    Hq, Hkv, D, BS = 8, 2, 128, 16
    p = prefill_case(3333, [500, 1500, 0], [100, 300, 130], Hq, Hkv, D, BS)
    rng = np.random.default_rng(3334)
    u = _directions(rng, Hkv, D)
    for i, (P, n) in enumerate(zip(p.prefix_lens, p.q_lens)):
        for t in range(int(P)):
            s = slot_for_position(p.block_tables[i], t, BS)
            p.k_cache[s // BS, s % BS] = bf16_bits_from_f32(_key(rng, u, t))
        q0 = int(p.cu_seqlens_q[i])
        for t in range(int(n)):
            p.k_new[q0 + t] = bf16_bits_from_f32(_key(rng, u, int(P) + t))
    p.q[:] = _queries(rng, u, p.total_q, Hq)
    say(f"[rescale] prefill prefixes {list(p.prefix_lens)} chunks {list(p.q_lens)}")
    out = torch.empty((p.total_q, Hq, D), dtype=torch.float32, device=dev)
    pa.paged_prefill(bf16(p.q, dev), bf16(p.k_new, dev), bf16(p.v_new, dev),
                     i32(p.cu_seqlens_q, dev), i32(p.block_tables, dev), i32(p.context_lens, dev),
                     out, k_cache=bf16(p.k_cache, dev), v_cache=bf16(p.v_cache, dev),
                     scale=p.scale, max_q_len=int(p.q_lens.max()))
    torch.cuda.synchronize()
    ref = oracle.paged_prefill(p.q, p.k_new, p.v_new, p.cu_seqlens_q, p.k_cache, p.v_cache,
                               p.block_tables, p.context_lens, np.float32(p.scale))
    err = np.abs(as_f64(out) - ref).max()
    say(f"[rescale] prefill: max|err| {err:.3e}")
    assert err <= ATOL
