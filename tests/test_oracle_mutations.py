"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one."""
import numpy as np
import pytest

import oracle
import oracle.block_manager as bm_oracle
import oracle.fp8 as fp8_oracle
import oracle.paged_attention as pa_oracle
from oracle_pins import PINS


def _caught(monkeypatch, name, replacement):
    if name.startswith("BlockManager."):
        monkeypatch.setattr(bm_oracle.BlockManager, name.split(".", 1)[1], replacement)
    for mod in (pa_oracle, fp8_oracle, bm_oracle, oracle):
        if hasattr(mod, name):
            monkeypatch.setattr(mod, name, replacement)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


def _softmax_no_scale(q_rows, K, V, scale, mask=None):
    s = q_rows @ K.T
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p @ V) / p.sum(axis=1, keepdims=True)


def _softmax_sign(q_rows, K, V, scale, mask=None):
    s = -(q_rows @ K.T) * float(scale)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p @ V) / p.sum(axis=1, keepdims=True)


def _softmax_values_are_keys(q_rows, K, V, scale, mask=None):
    s = (q_rows @ K.T) * float(scale)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p @ K) / p.sum(axis=1, keepdims=True)


def _softmax_unnormalised(q_rows, K, V, scale, mask=None):
    s = (q_rows @ K.T) * float(scale)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return p @ V


def _unpage_swapped(cache, table_row, n):
    bs = cache.shape[1]
    j = np.arange(int(n))
    return cache[np.asarray(table_row, np.int64)[j % len(table_row) if len(table_row) else j],
                 (j // max(len(table_row), 1)) % bs]


def _unpage_offset_by_one(cache, table_row, n):
    bs = cache.shape[1]
    j = np.arange(int(n)) + 1
    return cache[np.asarray(table_row, np.int64)[np.minimum(j // bs, len(table_row) - 1)], j % bs]


def _store_next_slot(k, v, slot_mapping, k_cache, v_cache):
    shifted = np.where(np.asarray(slot_mapping) >= 0, np.asarray(slot_mapping) + 1, -1)
    shifted = np.minimum(shifted, k_cache.shape[0] * k_cache.shape[1] - 1)
    return ORIGINAL_STORE(k, v, shifted, k_cache, v_cache)


ORIGINAL_STORE = pa_oracle.kvcache_store
ORIGINAL_ENCODE = fp8_oracle.e4m3_encode


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    nudged = x + np.sign(x) * np.abs(x) * 1e-12  # pushes exact ties upward in magnitude
    return ORIGINAL_ENCODE(nudged)


def _encode_no_saturation(x):
    x = np.asarray(x, dtype=np.float64)
    code = ORIGINAL_ENCODE(x)
    return np.where(np.abs(x) > 448.0, np.uint8(0x7F) | (code & 0x80), code).astype(np.uint8)


def _encode_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    vals = fp8_oracle.E4M3_TABLE[:0x7F]
    lo = np.clip(np.searchsorted(vals, np.minimum(a, 448.0), side="right") - 1, 0, 0x7E)
    return (lo.astype(np.uint8) | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)

def _encode_nan_unsigned(x):
    x = np.asarray(x, dtype=np.float64)
    code = ORIGINAL_ENCODE(x)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def _quantize_f64_division(bits_bf16, scale):
    x = (np.asarray(bits_bf16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return fp8_oracle.e4m3_encode(x.astype(np.float64) / np.float64(np.float32(scale)))


ORIGINAL_PREFILL_FP8 = fp8_oracle.paged_prefill_fp8


def _prefill_fp8_swapped_scales(q, cu, kc8, vc8, bt, ctx, scale, k_scale, v_scale):
    return ORIGINAL_PREFILL_FP8(q, cu, kc8, vc8, bt, ctx, scale, v_scale, k_scale)


def _prefill_fp8_sees_whole_chunk(q, cu, kc8, vc8, bt, ctx, scale, k_scale, v_scale):
    # every chunk token treated as the last one: no causal mask inside the chunk
    out = np.zeros(q.shape, dtype=np.float64)
    cu = np.asarray(cu, dtype=np.int64)
    for i in range(cu.shape[0] - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        for t in range(a, b):
            out[t] = oracle.paged_decode_fp8(q[t:t + 1], kc8, vc8, bt[i:i + 1],
                                             np.array([int(ctx[i])], np.int32), scale, k_scale,
                                             v_scale)[0]
    return out


ORIGINAL_HASH = bm_oracle.block_hash
ORIGINAL_ALLOCATE = bm_oracle.BlockManager.allocate
ORIGINAL_APPEND = bm_oracle.BlockManager.append
ORIGINAL_DEALLOCATE = bm_oracle.BlockManager.deallocate


def _fnv_wrong_prime(data, h=bm_oracle.FNV_OFFSET):
    for b in data:
        h = ((h ^ b) * 0x100000001B5) & bm_oracle.MASK64
    return h


class _Loose(list):
    """A token list that never differs from another: the cache-miss token compare always passes."""

    def __ne__(self, other):
        return False


def _allocate_without_token_compare(self, seq_id, tokens):
    for blk in self.blocks:
        blk.token_ids = _Loose(blk.token_ids)
    try:
        return ORIGINAL_ALLOCATE(self, seq_id, tokens)
    finally:
        for blk in self.blocks:
            blk.token_ids = list(blk.token_ids)


def _allocate_no_ref_on_hit(self, seq_id, tokens):
    before = [b.ref_count for b in self.blocks]
    n = ORIGINAL_ALLOCATE(self, seq_id, tokens)
    for b, r in zip(self.blocks, before):
        if r > 0 and b.ref_count == r + 1:
            b.ref_count = r
    return n


def _append_opens_late(self, seq_id, token):
    seq = self.seqs[seq_id]
    seq.token_ids.append(int(token))
    n, bs = len(seq.token_ids), self.block_size
    if n % bs == 0 and n // bs >= len(seq.block_table):
        seq.block_table.append(self._take(self.free[0]).block_id)


def _deallocate_first_block_first(self, seq_id):
    seq = self.seqs.pop(seq_id)
    for bid in seq.block_table:
        blk = self.blocks[bid]
        blk.ref_count -= 1
        if blk.ref_count == 0:
            self.used.discard(bid)
            self.free.append(bid)


MUTATIONS = {
    "bm_hash_wrong_prime": ("fnv1a64", _fnv_wrong_prime),
    "bm_hash_ignores_prefix": ("block_hash", lambda t, p, b=64: ORIGINAL_HASH(t, -1, b)),
    "bm_no_token_compare": ("BlockManager.allocate", _allocate_without_token_compare),
    "bm_no_ref_on_hit": ("BlockManager.allocate", _allocate_no_ref_on_hit),
    "bm_append_opens_late": ("BlockManager.append", _append_opens_late),
    "bm_free_first_block_first": ("BlockManager.deallocate", _deallocate_first_block_first),
    "gqa_modulo": ("kv_head_for", lambda h, g: h % max(1, g) if g > 1 else h // g),
    "causal_excludes_self": ("visible", lambda t, j, P: j < P + t),
    "causal_ignores_prefix": ("visible", lambda t, j, P: j <= t + 0 * P),
    "no_mask": ("visible", lambda t, j, P: (j >= 0) | (t >= 0)),
    "scale_dropped": ("softmax_attention", _softmax_no_scale),
    "score_sign": ("softmax_attention", _softmax_sign),
    "values_are_keys": ("softmax_attention", _softmax_values_are_keys),
    "not_normalised": ("softmax_attention", _softmax_unnormalised),
    "unpage_swapped_axes": ("unpage", _unpage_swapped),
    "unpage_off_by_one": ("unpage", _unpage_offset_by_one),
    "store_next_slot": ("kvcache_store", _store_next_slot),
    "e4m3_ties_away": ("e4m3_encode", _encode_ties_away),
    "e4m3_no_saturation": ("e4m3_encode", _encode_no_saturation),
    "e4m3_truncates": ("e4m3_encode", _encode_truncate),
    "e4m3_nan_loses_sign": ("e4m3_encode", _encode_nan_unsigned),
    "fp8_quant_divides_in_float64": ("quantize", _quantize_f64_division),
    "e4m3_bias_8":("e4m3_decode", lambda c: fp8_oracle.E4M3_TABLE[np.asarray(c, np.uint8)] / 2.0),
    "fp8_dequant_ignores_scale": ("dequantize", lambda c, s: fp8_oracle.e4m3_decode(c)),
    "fp8_quant_multiplies": ("quantize", lambda b, s: fp8_oracle.e4m3_encode(
        oracle.bf16_to_f64(b) * np.float32(s))),
    "fp8_prefill_swapped_scales": ("paged_prefill_fp8", _prefill_fp8_swapped_scales),
    "fp8_prefill_not_causal": ("paged_prefill_fp8", _prefill_fp8_sees_whole_chunk),
    "bf16_shift_8": ("bf16_to_f64", lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 8)
                     .view(np.float32).astype(np.float64)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    with np.errstate(all="ignore"):
        failed = _caught(monkeypatch, attr, fn)
    assert failed, f"no pin caught the planted mistake {name}"
