"""CPU oracle of the FP8 KV cache (test infrastructure only; see the package docstring).

The VLLM 0.7.3 source article (§5.3, KV cache precision) stores the KV cache in
FP8 while keeping the attention output in high precision.  The page names no
format or scaling; the readings taken here:

* codes are OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals, no infinities, NaN = S.1111.111, largest finite
  magnitude 448;
* one scale per tensor (``k_scale``, ``v_scale``): a value x is stored as
  ``code = E4M3(x / scale)`` and read back as ``decode(code) * scale``;
* ``x / scale`` is computed in float32, then rounded to the nearest E4M3 value
  with ties to even; magnitudes beyond 448 saturate to 448 and NaN stays NaN
  (sign kept).

Attention on an FP8 cache is the ordinary attention of ``oracle.paged_attention``
applied to the decoded-and-scaled K and V.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import bf16_to_f64, kv_head_for, softmax_attention, unpage, visible

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Exact value of one E4M3 code (NaN for S.1111.111)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


#: Values of all 256 codes.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes in increasing order of value: 0x00 .. 0x7E.
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of uint8 codes."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code (ties to even mantissa), saturating at 448; NaN -> S.1111.111."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # index of the largest representable value <= a, then pick the nearer neighbour
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def quantize(bits_bf16, scale: float) -> np.ndarray:
    """E4M3 codes of bf16 values divided by ``scale`` (the division in float32)."""
    x = (np.asarray(bits_bf16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    q = (x / np.float32(scale)).astype(np.float32)
    return e4m3_encode(q.astype(np.float64))


def dequantize(codes, scale: float) -> np.ndarray:
    """Exact float64 ``decode(code) * scale``."""
    return e4m3_decode(codes) * np.float64(np.float32(scale))


def kvcache_store_fp8(k, v, slot_mapping, k_cache8, v_cache8, k_scale, v_scale):
    """Quantize row t of k/v into slot ``slot_mapping[t]`` of copies of the uint8 caches."""
    kc = np.array(k_cache8, copy=True)
    vc = np.array(v_cache8, copy=True)
    block_size = kc.shape[1]
    kq = quantize(k, k_scale)
    vq = quantize(v, v_scale)
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        kc[blk, off] = kq[t]
        vc[blk, off] = vq[t]
    return kc, vc


def paged_decode_fp8(q, k_cache8, v_cache8, block_tables, context_lens, scale, k_scale,
                     v_scale) -> np.ndarray:
    """Decode over an FP8 cache: attention on the dequantized K and V; ``[B, Hq, D]`` float64."""
    B, Hq, D = q.shape
    Hkv = k_cache8.shape[2]
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for i in range(B):
        n = int(context_lens[i])
        if n == 0:
            continue
        K = dequantize(unpage(k_cache8, block_tables[i], n), k_scale)
        V = dequantize(unpage(v_cache8, block_tables[i], n), v_scale)
        for h in range(Hq):
            g = kv_head_for(h, group)
            qh = bf16_to_f64(q[i, h])[None, :]
            out[i, h] = softmax_attention(qh, K[:, g, :], V[:, g, :], scale)[0]
    return out


def paged_prefill_fp8(q, cu_seqlens_q, k_cache8, v_cache8, block_tables, context_lens, scale,
                      k_scale, v_scale) -> np.ndarray:
    """Prefix-hit prefill over an FP8 cache; ``[Tq, Hq, D]`` float64.

    The chunk's own tokens are already in the cache (stored before attention, as
    the store-then-attend order of a step has it), so every key ``0 .. ctx-1`` of
    sequence ``i`` is read through its block table and dequantized; chunk token
    ``t`` sits at position ``P + t`` with ``P = context_lens[i] - q_len_i`` and
    sees keys ``0 .. P + t``.
    """
    Tq, Hq, D = q.shape
    Hkv = k_cache8.shape[2]
    group = Hq // Hkv
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for i in range(cu.shape[0] - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        n = b - a
        if n == 0:
            continue
        ctx = int(context_lens[i])
        P = ctx - n
        K = dequantize(unpage(k_cache8, block_tables[i], ctx), k_scale)
        V = dequantize(unpage(v_cache8, block_tables[i], ctx), v_scale)
        mask = visible(np.arange(n)[:, None], np.arange(ctx)[None, :], P)
        for h in range(Hq):
            g = kv_head_for(h, group)
            Qh = bf16_to_f64(q[a:b, h])
            out[a:b, h] = softmax_attention(Qh, K[:, g, :], V[:, g, :], scale, mask)
    return out
