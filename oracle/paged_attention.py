"""Plain CPU definition of the paged-KV attention hot path (float64, NumPy).

Test infrastructure only: see the package docstring.

What is computed, and where the pages state it:

* KV store: every new token's K and V row is written into the flat cache slot
  its ``slot_mapping`` entry names; only new (uncached) tokens get a slot, and
  padded rows carry a sentinel (MinivLLM guide "vLLM 技术路线", Step 4 §4.4
  allocate_kv_cache and §4.5 prepare_prefill/prepare_decode; §4.6 run_model
  for the sentinels).  Slot ``s`` is offset ``s mod block_size`` of block
  ``s div block_size``: §4.5 forms a slot as ``block_id * block_size +
  offset``.
* Un-paging: logical token ``j`` of a sequence lives in physical block
  ``block_table[j div block_size]`` at offset ``j mod block_size`` (MinivLLM
  guide §4.5, a block is ``kv_cache[..., b*bs:(b+1)*bs, ...]``; VLLM 0.7.3
  source article §3.1, the logical -> physical block table).
* Attention: paging changes only where K and V are stored, not the result.
  The v0 engine of "Engine 推理引擎" (§3 generate, §5 v0 scope) recomputes
  the whole sequence every step without a cache; a cached step must give the
  same softmax(q K^T * scale) V over all tokens so far.  Decode and the
  prefix-hit prefill both read the paged cache through ``block_table``
  ("Nano-vLLM源码学习(2)", §2 Config, the paged flash-attn call).

Readings where the pages are silent (each also listed in the design notes):
query head ``h`` uses KV head ``h // (Hq / Hkv)``; ``context_lens`` counts all
keys including the token(s) being processed; ``context_lens == 0`` marks a
padded decode row whose output is zero; a prefill chunk of ``n`` tokens sits at
the end of its sequence, so chunk token ``t`` sees keys ``0 .. P + t`` with
``P = context_len - n``; the scale multiplies the exact dot product.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact float64 value of raw bfloat16 bit patterns (the top half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def kvcache_store(k, v, slot_mapping, k_cache, v_cache):
    """Write row ``t`` of ``k``/``v`` into slot ``slot_mapping[t]`` of copies of the caches.

    Negative slots are padding and write nothing.  The copy is bit for bit
    (``uint16`` patterns), so stored rows are exactly the inputs.
    Returns ``(k_cache', v_cache')``.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    block_size = kc.shape[1]
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        kc[blk, off] = k[t]
        vc[blk, off] = v[t]
    return kc, vc


def unpage(cache, table_row, n: int) -> np.ndarray:
    """Logical tokens ``0 .. n-1`` of one sequence, ``[n, Hkv, D]``, gathered via its block table."""
    block_size = cache.shape[1]
    j = np.arange(int(n))
    blocks = np.asarray(table_row, dtype=np.int64)[j // block_size]
    return cache[blocks, j % block_size]


def kv_head_for(h: int, group: int) -> int:
    """KV head serving query head ``h`` when ``group`` query heads share one KV head."""
    return h // group


def visible(t, j, prefix_len: int):
    """Whether chunk token ``t`` (absolute position ``prefix_len + t``) may attend to key ``j``.

    Works elementwise on broadcastable integer arrays.
    """
    return j <= prefix_len + t


def softmax_attention(q_rows, K, V, scale, mask=None) -> np.ndarray:
    """softmax(q_rows K^T * scale) V row by row; ``mask[r, j]`` False removes key ``j`` for row ``r``."""
    s = (q_rows @ K.T) * float(scale)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale) -> np.ndarray:
    """One query token per sequence over its paged context; ``[B, Hq, D]`` float64.

    ``q`` is ``[B, Hq, D]`` bf16 bits, the caches ``[NB, BS, Hkv, D]`` bf16 bits,
    ``block_tables`` ``[B, MBS]``, ``context_lens`` ``[B]`` (0: padded row, output 0).
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for i in range(B):
        n = int(context_lens[i])
        if n == 0:
            continue
        K = bf16_to_f64(unpage(k_cache, block_tables[i], n))
        V = bf16_to_f64(unpage(v_cache, block_tables[i], n))
        for h in range(Hq):
            g = kv_head_for(h, group)
            qh = bf16_to_f64(q[i, h])[None, :]
            out[i, h] = softmax_attention(qh, K[:, g, :], V[:, g, :], scale)[0]
    return out


def paged_prefill(q, k_new, v_new, cu_seqlens_q, k_cache, v_cache, block_tables, context_lens,
                  scale) -> np.ndarray:
    """Prefix-hit prefill: each chunk attends to its cached prefix plus itself, causally.

    ``q`` is ``[Tq, Hq, D]``, ``k_new``/``v_new`` ``[Tq, Hkv, D]`` (bf16 bits) flattened
    along ``cu_seqlens_q``; the first ``context_lens[i] - q_len_i`` keys of sequence
    ``i`` come from the paged cache, the rest from ``k_new``/``v_new``.
    Returns ``[Tq, Hq, D]`` float64.
    """
    Tq, Hq, D = q.shape
    Hkv = k_new.shape[1]
    group = Hq // Hkv
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for i in range(cu.shape[0] - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        n = b - a
        if n == 0:
            continue
        P = int(context_lens[i]) - n
        K = np.concatenate([bf16_to_f64(unpage(k_cache, block_tables[i], P)),
                            bf16_to_f64(k_new[a:b])])
        V = np.concatenate([bf16_to_f64(unpage(v_cache, block_tables[i], P)),
                            bf16_to_f64(v_new[a:b])])
        mask = visible(np.arange(n)[:, None], np.arange(P + n)[None, :], P)
        for h in range(Hq):
            g = kv_head_for(h, group)
            Qh = bf16_to_f64(q[a:b, h])
            out[a:b, h] = softmax_attention(Qh, K[:, g, :], V[:, g, :], scale, mask)
    return out
