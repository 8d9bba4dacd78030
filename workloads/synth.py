"""Seeded generators for the five paged-attention workloads and for small cases.

Every value is drawn from ``numpy.random.default_rng(seed)`` as float32 N(0, 1)
and rounded to bfloat16 (round to nearest, ties to even).  bfloat16 tensors are
carried as their raw ``uint16`` bit patterns; the GPU side views them as
``torch.bfloat16`` and the oracle decodes them itself.

Layout conventions (the same ones the library documents):

* K and V caches are separate pools ``[num_blocks, block_size, num_kv_heads,
  head_dim]``: the token axis of a block comes before the head axes, as in the
  MinivLLM guide "vLLM 技术路线", Step 4 §4.5 (a block is sliced as
  ``kv_cache[..., b*bs:(b+1)*bs, ...]``).
* ``block_tables`` is ``int32 [B, max_blocks_per_seq]`` padded with -1, one
  row of physical block ids per sequence (same guide §4.5, "block_tables";
  VLLM 0.7.3 source article §3.1, logical -> physical block table).
* Slots not holding a valid token are poisoned with bfloat16 NaN so that any
  read of an unused slot shows up in the results.

Draw order per workload, from ``default_rng(seed)``: context lengths, sharing
groups, the physical block permutation, then q, k_new, v_new.  Pool contents
come from one child stream per sharing group and per sequence (K before V,
logical order), seeded by ``SeedSequence([seed, role, index])``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BF16_NAN = 0x7FC0

#: Fixed seeds of the five named workloads.
CONFIG_SEEDS = {1: 8601, 2: 8602, 3: 8603, 4: 8604, 5: 8605}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    u = x.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def cu_seqlens_from_lens(lens: Sequence[int]) -> np.ndarray:
    """Cumulative boundaries ``[0, l0, l0+l1, ...]`` of a flattened varlen batch.

    The MinivLLM guide "vLLM 技术路线", Step 4 §4.5 (prepare_prefill) draws
    ``cu_seqlens_q = [0, 3, 5, 9]`` for three sequences of lengths 3, 2, 4.
    """
    out = np.zeros(len(lens) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return out


def slot_for_position(table_row: Sequence[int], pos: int, block_size: int) -> int:
    """Flat cache slot of logical token ``pos`` of a sequence.

    The new-token slot of a decode step is ``block_table[-1] * block_size +
    last_block_num_tokens - 1`` (MinivLLM guide, Step 4 §4.5 prepare_decode);
    for an arbitrary position it is the block holding it times the block size
    plus the offset inside that block.
    """
    blk, off = divmod(int(pos), int(block_size))
    return int(table_row[blk]) * int(block_size) + off


def _ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


@dataclass
class _Pool:
    block_tables: np.ndarray  # int32 [B, MBS], -1 padded
    num_blocks: int
    max_blocks_per_seq: int
    shared_groups: List[List[int]]
    shared_blocks: List[int]  # per group: number of leading shared blocks


def _allocate_tables(rng, needed_blocks, shared_groups, shared_blocks, num_blocks,
                     nb_factor, max_blocks_per_seq) -> _Pool:
    """Assign physical blocks from a seeded permutation of the pool.

    Shared leading blocks of a group are taken once and referenced by every
    member (prefix sharing: MinivLLM guide, Step 3 §3.2, reference-counted
    blocks reused through the prefix hash).
    """
    B = len(needed_blocks)
    member_of = {}
    for g, members in enumerate(shared_groups):
        for m in members:
            member_of[m] = g
    unique = int(sum(needed_blocks)) - int(sum((len(m) - 1) * s for m, s in
                                                zip(shared_groups, shared_blocks)))
    if num_blocks is None:
        num_blocks = int(np.ceil(nb_factor * unique)) if nb_factor else unique
    if unique > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {unique} blocks")
    mbs = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(needed_blocks))
    if max(needed_blocks) > mbs:
        raise ValueError("max_blocks_per_seq too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    group_ids = []
    for s in shared_blocks:
        group_ids.append(perm[cursor:cursor + s])
        cursor += s
    tables = np.full((B, mbs), -1, dtype=np.int32)
    for i in range(B):
        row = []
        if i in member_of:
            row.extend(int(x) for x in group_ids[member_of[i]])
        own = needed_blocks[i] - len(row)
        row.extend(int(x) for x in perm[cursor:cursor + own])
        cursor += own
        tables[i, :len(row)] = row
    return _Pool(tables, int(num_blocks), int(mbs), [list(m) for m in shared_groups],
                 list(shared_blocks))


def _fill_blocks(pool: np.ndarray, table_row, first_pos: int, rows: np.ndarray, block_size: int):
    """Place ``rows`` (logical positions ``first_pos ..``) into their pool blocks."""
    n = rows.shape[0]
    pos = first_pos
    while pos < first_pos + n:
        blk = pos // block_size
        off = pos - blk * block_size
        take = min(block_size - off, first_pos + n - pos)
        pool[int(table_row[blk]), off:off + take] = rows[pos - first_pos:pos - first_pos + take]
        pos += take


def _child_rng(seed: int, role: int, index: int) -> np.random.Generator:
    """Independent stream for one group's or one sequence's cache contents."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(role), int(index)]))


def _workers() -> int:
    try:
        import os
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except Exception:  # pragma: no cover - non-Linux hosts
        return 4


def _fill_contents(seed, pool_k, pool_v, tables, cached_lens, shared_groups, shared_blocks,
                   block_size, Hkv, D, keep_logical):
    """Draw K/V for the cached positions ``0 .. cached_lens[i]-1`` of each sequence.

    Group ``g``'s shared prefix comes from stream ``(seed, 1, g)`` and sequence
    ``i``'s own tokens from stream ``(seed, 2, i)`` (K, then V), so the draws do
    not depend on the order in which the worker threads run.  Shared blocks are
    written once, by their group; every other block belongs to one sequence.
    """
    from concurrent.futures import ThreadPoolExecutor

    B = len(cached_lens)
    member_of = {}
    for g, members in enumerate(shared_groups):
        for m in members:
            member_of[m] = g
        if shared_blocks[g] * block_size > min(int(cached_lens[m]) for m in members):
            raise ValueError("shared prefix longer than the cached context")

    def group_task(g):
        r = _child_rng(seed, 1, g)
        n_sh = shared_blocks[g] * block_size
        k_sh = _normal_bf16(r, (n_sh, Hkv, D))
        v_sh = _normal_bf16(r, (n_sh, Hkv, D))
        _fill_blocks(pool_k, tables[shared_groups[g][0]], 0, k_sh, block_size)
        _fill_blocks(pool_v, tables[shared_groups[g][0]], 0, v_sh, block_size)
        return (k_sh, v_sh) if keep_logical else None

    def seq_task(i):
        r = _child_rng(seed, 2, i)
        n = int(cached_lens[i])
        start = shared_blocks[member_of[i]] * block_size if i in member_of else 0
        k_own = _normal_bf16(r, (n - start, Hkv, D))
        v_own = _normal_bf16(r, (n - start, Hkv, D))
        _fill_blocks(pool_k, tables[i], start, k_own, block_size)
        _fill_blocks(pool_v, tables[i], start, v_own, block_size)
        return (k_own, v_own) if keep_logical else None

    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        prefixes = list(ex.map(group_task, range(len(shared_groups))))
        owns = list(ex.map(seq_task, range(B)))
    if not keep_logical:
        return None, None
    logical_k, logical_v = [], []
    for i in range(B):
        k_own, v_own = owns[i]
        if i in member_of:
            k_sh, v_sh = prefixes[member_of[i]]
            k_own, v_own = np.concatenate([k_sh, k_own]), np.concatenate([v_sh, v_own])
        logical_k.append(k_own)
        logical_v.append(v_own)
    return logical_k, logical_v


@dataclass
class DecodeInputs:
    """One decode step: store one new K/V row per sequence, then attend.

    ``k_cache``/``v_cache`` hold positions ``0 .. ctx-2`` of every sequence;
    position ``ctx-1`` (the token being decoded) arrives in ``k_new``/``v_new``
    and is written by the store through ``slot_mapping``.  Rows with
    ``context_lens == 0`` are padding: slot -1, output 0.
    """
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    context_lens: np.ndarray
    block_tables: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    shared_groups: List[List[int]] = field(default_factory=list)
    shared_blocks: List[int] = field(default_factory=list)
    logical_k: Optional[list] = None
    logical_v: Optional[list] = None

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    def kv_bytes(self) -> int:
        """Bytes of K and V one decode call must read (logical, shared blocks counted per reader)."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * 2

    def unique_kv_bytes(self) -> int:
        nb = 0
        seen = set()
        for i, n in enumerate(self.context_lens):
            for j in range(_ceil_div(int(n), self.block_size)):
                b = int(self.block_tables[i, j])
                if b in seen:
                    continue
                seen.add(b)
                nb += min(self.block_size, int(n) - j * self.block_size)
        return nb * 2 * self.num_kv_heads * self.head_dim * 2


@dataclass
class PrefillInputs:
    """One prefix-hit prefill chunk.

    Sequence ``i`` has ``prefix_lens[i]`` cached tokens in the pool and
    ``q_lens[i]`` new tokens in ``q``/``k_new``/``v_new`` (flattened along
    ``cu_seqlens_q``); ``context_lens = prefix_lens + q_lens``.
    ``slot_mapping`` gives the slots of the new tokens, for the store.
    """
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    prefix_lens: np.ndarray
    q_lens: np.ndarray
    context_lens: np.ndarray
    cu_seqlens_q: np.ndarray
    block_tables: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    logical_k: Optional[list] = None
    logical_v: Optional[list] = None

    @property
    def batch(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    def flops(self) -> int:
        """Multiply-add flops of QK^T and PV over the unmasked (query, key) pairs."""
        pairs = 0
        for p, n in zip(self.prefix_lens, self.q_lens):
            p, n = int(p), int(n)
            pairs += n * p + n * (n + 1) // 2
        return 4 * self.num_q_heads * self.head_dim * pairs


def decode_case(seed: int, context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, *, num_blocks: Optional[int] = None, nb_factor: Optional[float] = None,
                max_blocks_per_seq: Optional[int] = None, shared_groups=(), shared_blocks=(),
                keep_logical: bool = False, name: str = "case", rng=None) -> DecodeInputs:
    """Build a decode step for given context lengths (drawn from ``seed`` unless ``rng`` is given)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    ctx = np.asarray(context_lens, dtype=np.int32)
    B = ctx.shape[0]
    Hkv, D, BS = num_kv_heads, head_dim, block_size
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    needed = [_ceil_div(int(n), BS) for n in ctx]
    pool = _allocate_tables(rng, needed, list(shared_groups), list(shared_blocks), num_blocks,
                            nb_factor, max_blocks_per_seq)
    k_cache = np.full((pool.num_blocks, BS, Hkv, D), BF16_NAN, dtype=np.uint16)
    v_cache = np.full_like(k_cache, BF16_NAN)
    cached = np.maximum(ctx.astype(np.int64) - 1, 0)
    lk, lv = _fill_contents(seed, k_cache, v_cache, pool.block_tables, cached, pool.shared_groups,
                            pool.shared_blocks, BS, Hkv, D, keep_logical)
    q = _normal_bf16(rng, (B, num_q_heads, D))
    k_new = _normal_bf16(rng, (B, Hkv, D))
    v_new = _normal_bf16(rng, (B, Hkv, D))
    slots = np.full(B, -1, dtype=np.int32)
    for i in range(B):
        if ctx[i] > 0:
            slots[i] = slot_for_position(pool.block_tables[i], int(ctx[i]) - 1, BS)
    return DecodeInputs(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=Hkv,
                        head_dim=D, block_size=BS, num_blocks=pool.num_blocks,
                        max_blocks_per_seq=pool.max_blocks_per_seq, scale=float(1.0 / np.sqrt(D)),
                        context_lens=ctx, block_tables=pool.block_tables, k_cache=k_cache,
                        v_cache=v_cache, q=q, k_new=k_new, v_new=v_new, slot_mapping=slots,
                        shared_groups=pool.shared_groups, shared_blocks=pool.shared_blocks,
                        logical_k=lk, logical_v=lv)


def prefill_case(seed: int, prefix_lens, q_lens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, *, num_blocks: Optional[int] = None,
                 max_blocks_per_seq: Optional[int] = None, keep_logical: bool = False,
                 name: str = "case", rng=None) -> PrefillInputs:
    """Build a prefix-hit prefill chunk for given prefix and chunk lengths."""
    rng = np.random.default_rng(seed) if rng is None else rng
    P = np.asarray(prefix_lens, dtype=np.int32)
    n = np.asarray(q_lens, dtype=np.int32)
    if P.shape != n.shape:
        raise ValueError("prefix_lens and q_lens must have the same length")
    Hkv, D, BS = num_kv_heads, head_dim, block_size
    ctx = (P.astype(np.int64) + n).astype(np.int32)
    needed = [_ceil_div(int(c), BS) for c in ctx]
    pool = _allocate_tables(rng, needed, [], [], num_blocks, None, max_blocks_per_seq)
    k_cache = np.full((pool.num_blocks, BS, Hkv, D), BF16_NAN, dtype=np.uint16)
    v_cache = np.full_like(k_cache, BF16_NAN)
    lk, lv = _fill_contents(seed, k_cache, v_cache, pool.block_tables, P, [], [], BS, Hkv, D,
                            keep_logical)
    cu = cu_seqlens_from_lens(n)
    Tq = int(cu[-1])
    q = _normal_bf16(rng, (Tq, num_q_heads, D))
    k_new = _normal_bf16(rng, (Tq, Hkv, D))
    v_new = _normal_bf16(rng, (Tq, Hkv, D))
    slots = np.empty(Tq, dtype=np.int32)
    for i in range(P.shape[0]):
        for t in range(int(n[i])):
            slots[cu[i] + t] = slot_for_position(pool.block_tables[i], int(P[i]) + t, BS)
    return PrefillInputs(name=name, seed=seed, num_q_heads=num_q_heads, num_kv_heads=Hkv,
                         head_dim=D, block_size=BS, num_blocks=pool.num_blocks,
                         max_blocks_per_seq=pool.max_blocks_per_seq, scale=float(1.0 / np.sqrt(D)),
                         prefix_lens=P, q_lens=n, context_lens=ctx, cu_seqlens_q=cu,
                         block_tables=pool.block_tables, k_cache=k_cache, v_cache=v_cache, q=q,
                         k_new=k_new, v_new=v_new, slot_mapping=slots, logical_k=lk, logical_v=lv)


def mixed_case(seed: int, chunk_prefix_lens, chunk_q_lens, decode_context_lens, num_q_heads: int,
               num_kv_heads: int, head_dim: int, block_size: int, *,
               num_blocks: Optional[int] = None, max_blocks_per_seq: Optional[int] = None,
               name: str = "mixed") -> PrefillInputs:
    """A batch of prefill chunks followed by one-token decode rows, in one pool.

    A decode row of context ``c`` is a chunk of one token over a prefix of ``c - 1``; the
    returned inputs list the chunks first, then the decode sequences.
    """
    dctx = np.asarray(decode_context_lens, dtype=np.int32)
    P = np.concatenate([np.asarray(chunk_prefix_lens, np.int32), dctx - 1]).astype(np.int32)
    n = np.concatenate([np.asarray(chunk_q_lens, np.int32), np.ones_like(dctx)]).astype(np.int32)
    return prefill_case(seed, P, n, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq, name=name)


def _config4_sharing(rng, ctx, n_groups=13, group_size=4, block_size=256):
    eligible = np.nonzero(ctx > block_size)[0]
    chosen = rng.choice(eligible, size=n_groups * group_size, replace=False)
    groups = [sorted(int(x) for x in chosen[g * group_size:(g + 1) * group_size])
              for g in range(n_groups)]
    blocks = [int((min(int(ctx[m]) for m in grp) - 1) // block_size) for grp in groups]
    return groups, blocks


def config(cfg_id: int, keep_logical: bool = False):
    """The five named workloads (decode for 1-4, prefix-hit prefill for 5).

    1. tiny decode: ctx {17, 64, 200, 255}; 2 q heads, 1 KV head, D 64, block 16, 64-block pool.
    2. Qwen3-0.6B-shaped decode: B 64, 16/8 heads, D 128, block 256, ctx U{128..4096}, 2048 blocks.
    3. 7B-shaped decode: B 256, 28/4 heads, D 128, block 16, ctx U{512..8192}, pool 1.2x needed.
    4. max-concurrency decode: B 512, 16/8 heads, D 128, block 256, ctx log-normal (median 600,
       sigma 1) clipped to [1, 4096]; 13 groups of 4 sequences share their leading full blocks.
    5. prefix-hit prefill: 16 sequences x 512 new tokens, prefix U{0..3584}, 16/8 heads, D 128,
       block 256, 2048 blocks.
    """
    seed = CONFIG_SEEDS[cfg_id]
    rng = np.random.default_rng(seed)
    if cfg_id == 1:
        ctx = np.array([17, 64, 200, 255], dtype=np.int32)
        return decode_case(seed, ctx, 2, 1, 64, 16, num_blocks=64, max_blocks_per_seq=16,
                           keep_logical=keep_logical, name="tiny_decode", rng=rng)
    if cfg_id == 2:
        ctx = rng.integers(128, 4096, size=64, endpoint=True).astype(np.int32)
        return decode_case(seed, ctx, 16, 8, 128, 256, num_blocks=2048, max_blocks_per_seq=16,
                           keep_logical=keep_logical, name="qwen3_0.6b_decode_b64", rng=rng)
    if cfg_id == 3:
        ctx = rng.integers(512, 8192, size=256, endpoint=True).astype(np.int32)
        return decode_case(seed, ctx, 28, 4, 128, 16, nb_factor=1.2, max_blocks_per_seq=512,
                           keep_logical=keep_logical, name="7b_decode_b256_bs16", rng=rng)
    if cfg_id == 4:
        raw = rng.lognormal(mean=np.log(600.0), sigma=1.0, size=512)
        ctx = np.clip(np.rint(raw), 1, 4096).astype(np.int32)
        groups, blocks = _config4_sharing(rng, ctx)
        return decode_case(seed, ctx, 16, 8, 128, 256, nb_factor=1.2, max_blocks_per_seq=16,
                           shared_groups=groups, shared_blocks=blocks, keep_logical=keep_logical,
                           name="maxconc_decode_b512", rng=rng)
    if cfg_id == 5:
        P = rng.integers(0, 3584, size=16, endpoint=True).astype(np.int32)
        n = np.full(16, 512, dtype=np.int32)
        return prefill_case(seed, P, n, 16, 8, 128, 256, num_blocks=2048, max_blocks_per_seq=16,
                            keep_logical=keep_logical, name="prefix_hit_prefill_16x512", rng=rng)
    raise ValueError(f"unknown workload {cfg_id}")
