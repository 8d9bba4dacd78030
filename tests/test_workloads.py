"""Structure of the seeded workloads (sizes, tables, sharing, slots); no attention arithmetic."""
import numpy as np
import pytest

from workloads import BF16_NAN, bf16_bits_from_f32, config, decode_case, prefill_case


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties up to 1+2^-6
    assert bf16_bits_from_f32(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]


def test_config1_matches_its_description():
    c = config(1)
    assert c.context_lens.tolist() == [17, 64, 200, 255]
    assert (c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, c.num_blocks) == (2, 1, 64, 16, 64)
    assert c.scale == 0.125
    used = c.block_tables[c.block_tables >= 0]
    assert len(used) == 2 + 4 + 13 + 16 and len(set(used.tolist())) == len(used)
    assert c.kv_bytes() == (17 + 64 + 200 + 255) * 2 * 1 * 64 * 2


def test_decode_slots_point_at_the_last_position():
    c = decode_case(2, [1, 16, 17, 33, 0], 2, 1, 64, 16, nb_factor=1.5)
    for i, n in enumerate(c.context_lens):
        if n == 0:
            assert c.slot_mapping[i] == -1
            continue
        blk = c.block_tables[i, (n - 1) // 16]
        assert c.slot_mapping[i] == blk * 16 + (n - 1) % 16
        # the slot to be written is still poisoned
        assert np.all(c.k_cache[blk, (n - 1) % 16] == BF16_NAN)


def test_prefill_case_layout():
    p = prefill_case(3, [0, 20, 7], [5, 16, 9], 4, 2, 64, 16)
    assert p.cu_seqlens_q.tolist() == [0, 5, 21, 30]
    assert p.context_lens.tolist() == [5, 36, 16]
    assert p.flops() == 4 * 4 * 64 * (5 * 6 // 2 + 16 * 20 + 16 * 17 // 2 + 9 * 7 + 9 * 10 // 2)
    # slots of the new tokens follow the prefix
    assert p.slot_mapping[5] == p.block_tables[1, 1] * 16 + 4


@pytest.mark.slow
def test_config4_sharing_never_writes_a_shared_block():
    c = config(4)
    assert c.batch == 512 and c.context_lens.min() >= 1 and c.context_lens.max() <= 4096
    assert len(c.shared_groups) == 13 and all(len(g) == 4 for g in c.shared_groups)
    shared = set()
    for grp, nb in zip(c.shared_groups, c.shared_blocks):
        assert nb >= 1
        rows = [tuple(c.block_tables[m, :nb]) for m in grp]
        assert len(set(rows)) == 1
        shared.update(rows[0])
    written = {int(s) // 256 for s in c.slot_mapping if s >= 0}
    assert not (written & shared)
    assert c.unique_kv_bytes() < c.kv_bytes()
