"""End to end on the GPU with the C++ block manager driving the index arrays: prefix-hit
prefills (shared and revived cached blocks) and fused store + decode steps, against the oracle
running the same steps with the oracle block manager.  Caches compared bit for bit."""
import hashlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_86_amd as pa
from gpu_util import as_f64, bf16, bits, device, i32, say
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu

ATOL = 1e-2
NB, BS, HQ, HKV, D, MBS = 96, 16, 8, 2, 128, 16
SCALE = np.float32(1 / np.sqrt(D))


def kv_rows(tokens, start, stop):
    """K and V of positions start..stop-1: a function of the token prefix up to each position,
    so that sequences sharing a prefix share its K/V (as a model's cache does)."""
    ks, vs = [], []
    for p in range(start, stop):
        h = hashlib.sha256(np.asarray(tokens[:p + 1], np.int64).tobytes()).digest()
        r = np.random.default_rng(int.from_bytes(h[:8], "little"))
        ks.append(bf16_bits_from_f32(r.standard_normal((HKV, D), dtype=np.float32)))
        vs.append(bf16_bits_from_f32(r.standard_normal((HKV, D), dtype=np.float32)))
    if not ks:
        return np.zeros((0, HKV, D), np.uint16), np.zeros((0, HKV, D), np.uint16)
    return np.stack(ks), np.stack(vs)


class Engine:
    def __init__(self, dev):
        self.dev = dev
        self.cm = pa.BlockManager(NB, BS)
        self.om = oracle.BlockManager(NB, BS)
        nan = np.full((NB, BS, HKV, D), 0x7FC0, np.uint16)
        self.kc, self.vc = bf16(nan, dev), bf16(nan, dev)
        self.okc, self.ovc = nan.copy(), nan.copy()
        self.rng = np.random.default_rng(77)
        self.tokens = {}

    def prefill(self, ids, prompts):
        for sid, toks in zip(ids, prompts):
            c1 = self.cm.allocate(sid, toks)
            c2 = self.om.allocate(sid, toks)
            assert c1 == c2
            self.tokens[sid] = list(toks)
        pre = self.cm.prepare_prefill(ids, MBS)
        kn, vn = [], []
        for sid in ids:
            n, cached, _ = self.cm.seq_info(sid)
            k, v = kv_rows(self.tokens[sid], cached, n)
            kn.append(k)
            vn.append(v)
        kn, vn = np.concatenate(kn), np.concatenate(vn)
        T = pre["total_q"]
        q = bf16_bits_from_f32(self.rng.standard_normal((T, HQ, D), dtype=np.float32))
        out = torch.empty((T, HQ, D), dtype=torch.float32, device=self.dev)
        # Store first: a sequence of this step may reuse blocks another one fills in this step
        # (its prefix is read from the cache, the new tokens from k_new / v_new).
        pa.kvcache_store(bf16(kn, self.dev), bf16(vn, self.dev), i32(pre["slot_mapping"], self.dev),
                         self.kc, self.vc)
        pa.paged_prefill(bf16(q, self.dev), bf16(kn, self.dev), bf16(vn, self.dev),
                         i32(pre["cu_seqlens_q"], self.dev), i32(pre["block_tables"], self.dev),
                         i32(pre["context_lens"], self.dev), out, k_cache=self.kc, v_cache=self.vc,
                         scale=float(SCALE), max_q_len=max(pre["max_q_len"], 1))
        # oracle: same arrays from the oracle manager
        oslots = [s for sid in ids for s in self.om.prefill_slots(sid)]
        assert oslots == pre["slot_mapping"].tolist()
        self.okc, self.ovc = oracle.kvcache_store(kn, vn, np.asarray(oslots, np.int32), self.okc,
                                                  self.ovc)
        ref = oracle.paged_prefill(q, kn, vn, pre["cu_seqlens_q"], self.okc, self.ovc,
                                   pre["block_tables"], pre["context_lens"], SCALE)
        err = np.abs(as_f64(out) - ref).max()
        say(f"[engine] prefill {ids}: {T} new tokens, max|err| {err:.3e}")
        assert err <= ATOL

    def decode_step(self, ids):
        for sid in ids:
            tok = int(self.rng.integers(0, 50))
            assert self.cm.can_append(sid) and self.om.can_append(sid)
            self.cm.append(sid, tok)
            self.om.append(sid, tok)
            self.tokens[sid].append(tok)
        slots, lens, tables = self.cm.prepare_decode(ids, MBS)
        assert slots.tolist() == [self.om.decode_slot(s) for s in ids]
        kn, vn = zip(*[kv_rows(self.tokens[s], len(self.tokens[s]) - 1, len(self.tokens[s]))
                       for s in ids])
        kn, vn = np.concatenate(kn), np.concatenate(vn)
        q = bf16_bits_from_f32(self.rng.standard_normal((len(ids), HQ, D), dtype=np.float32))
        out = torch.empty((len(ids), HQ, D), dtype=torch.float32, device=self.dev)
        pa.paged_decode_append(bf16(q, self.dev), bf16(kn, self.dev), bf16(vn, self.dev),
                               i32(slots, self.dev), self.kc, self.vc, i32(tables, self.dev),
                               i32(lens, self.dev), float(SCALE), out)
        self.okc, self.ovc = oracle.kvcache_store(kn, vn, slots, self.okc, self.ovc)
        ref = oracle.paged_decode(q, self.okc, self.ovc, tables, lens, SCALE)
        err = np.abs(as_f64(out) - ref).max()
        assert err <= ATOL
        return err

    def release(self, sid):
        self.cm.deallocate(sid)
        self.om.deallocate(sid)
        assert self.cm.free_list() == list(self.om.free)

    def check_pools(self):
        torch.cuda.synchronize()
        used = sorted({b for s in self.om.seqs.values() for b in s.block_table})
        assert np.array_equal(bits(self.kc)[used], self.okc[used])
        assert np.array_equal(bits(self.vc)[used], self.ovc[used])


def test_engine_prefix_cache_prefill_and_decode():
    dev = device()
    e = Engine(dev)
    base = list(range(1, 49))                       # 3 full blocks
    a = base + [101, 102, 103, 104, 105]
    b = base + [201, 202]
    c = list(range(300, 337))
    e.prefill([1, 2], [a, b])                        # 2 reuses the 3 blocks 1 fills in this step
    assert e.cm.seq_info(2)[1] == 48
    errs = [e.decode_step([1, 2]) for _ in range(12)]  # crosses a block boundary
    say(f"[engine] decode max|err| {max(errs):.3e}")
    e.check_pools()
    e.prefill([3], [c])
    e.release(1)                                     # 1's own blocks freed; shared ones stay
    e.prefill([4], [a + [106]])                      # hits the 3 shared blocks (still in use)
    assert e.cm.seq_info(4)[1] == 48
    for _ in range(20):
        e.decode_step([2, 3, 4])
    e.check_pools()
    e.release(2)
    c_now = list(e.tokens[3])
    e.release(3)                                     # 3's blocks are free but still cached
    e.prefill([5, 6, 7], [b + [203], base, c_now[:40]])
    assert e.cm.seq_info(6)[1] == 48                 # fully cached prompt: nothing to compute
    assert e.cm.seq_info(7)[1] == 32                 # two of 3's freed blocks taken back
    e.decode_step([4, 5, 6, 7])
    e.check_pools()
