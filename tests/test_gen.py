"""Checks of the seeded input generator (CPU only)."""
import numpy as np
import pytest

from workloads import make_config, make_custom, blocks_for, round_to_bits


def test_blocks_for_matches_full_plus_tail():
    # "N tokens = full chunks + tail" applied to 16-token blocks
    # (kvboost 0.6.0, "How it works", step 1: 1000 tokens at 128 -> 7 full + 104 tail)
    assert (1000 // 128, 1000 % 128) == (7, 104)
    assert blocks_for(1000) == 1000 // 16 + 1 == 63
    assert blocks_for(0) == 0 and blocks_for(16) == 1 and blocks_for(17) == 2


def test_round_to_bits_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    # bf16 has 7 fraction bits: 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 -> 1+2^-6
    assert list(round_to_bits(x, "bf16")) == [0x3F80, 0x3F80, 0x3F82, 0xC020]
    assert list(round_to_bits(x[:1], "fp16")) == [0x3C00]


def test_determinism_and_seed_dependence():
    a = make_custom(3, "bf16", 4, 2, 64, [40, 7], [5, 9])
    b = make_custom(3, "bf16", 4, 2, 64, [40, 7], [5, 9])
    c = make_custom(4, "bf16", 4, 2, 64, [40, 7], [5, 9])
    assert np.array_equal(a.k_pool, b.k_pool) and np.array_equal(a.q, b.q)
    assert not np.array_equal(a.q, c.q)


def test_tables_in_range_and_disjoint_except_sharing():
    w = make_custom(5, "fp16", 4, 2, 32, [64, 70, 33, 48], [3, 3, 3, 3], share="pairs")
    seen = {}
    for b in range(w.batch):
        n = blocks_for(int(w.prefix_lens[b]) + int(w.q_lens[b]))
        row = w.block_tables[b, :n]
        assert (row >= 0).all() and (row < w.num_blocks).all()
        for j, pb in enumerate(row):
            seen.setdefault(int(pb), []).append((b, j))
    for pb, users in seen.items():
        if len(users) > 1:
            # shared blocks are only leading full prefix blocks, same logical index
            js = {j for _, j in users}
            assert len(js) == 1
            j = js.pop()
            for b, _ in users:
                assert 16 * (j + 1) <= int(w.prefix_lens[b])


def test_slot_mapping_points_at_chunk_positions():
    w = make_custom(6, "bf16", 2, 1, 16, [20, 0], [15, 18])
    for b in range(2):
        for i in range(int(w.q_lens[b])):
            pos = int(w.prefix_lens[b]) + i
            s = int(w.slot_mapping[w.cu_q_lens[b] + i])
            assert s // 16 == w.block_tables[b][pos // 16] and s % 16 == pos % 16


def test_page_bytes_formula():
    # one page = block_size x heads x head_dim x 2 x dtype_bytes (kvstream 0.1.0, "Configuration")
    w = make_config("tiny")
    page = 16 * w.num_kv_heads * w.head_dim * 2 * 2
    assert w.k_pool[0].nbytes + w.v_pool[0].nbytes == page


def test_config_statistics():
    w = make_config("tiny")
    assert w.block_tables.shape == (1, 3) and w.head_dim == 64 and w.scale == 0.125
    assert w.prefix_lens.tolist() == [32] and w.q_lens.tolist() == [16]
    w = make_config("shared_prompt")
    assert (w.block_tables[:, :128] == w.block_tables[0, :128]).all()
    assert len(set(w.block_tables[:, 128:144].ravel().tolist())) == 8 * 16


@pytest.mark.parametrize("name,stats", [
    ("ragged_d96", (241746, 8327, 0.402)),
    ("ragged_d64", (307020, 7306, 0.465)),
])
def test_ragged_statistics(name, stats):
    w = make_config(name)
    assert int(w.prefix_lens.sum()) == stats[0]
    assert int(w.q_lens.sum()) == stats[1]
    assert (w.q_lens % 16 != 0).all() and w.q_lens.min() >= 1 and w.q_lens.max() <= 512
    assert round(w.shared_fraction, 3) == stats[2]


def test_channel_scales_hand_values():
    """The K scales picked from example tokens: per (head, channel) the largest |k| over
    the tokens divided by the largest code, in float32 (values chosen so the quotients
    are exact)."""
    from workloads import channel_scales
    k = np.zeros((3, 2, 4), np.float32)
    k[0, 0] = [127.0, -254.0, 0.0, 63.5]
    k[1, 0] = [-12.0, 100.0, 0.0, -63.5]
    k[2, 1] = [7.0, -3.5, 0.875, 0.0]
    s8 = channel_scales(k)
    assert s8.dtype == np.float32
    assert s8[0].tolist() == [1.0, 2.0, 0.0, 0.5]
    assert s8[1].tolist() == [np.float32(7.0) / np.float32(127), np.float32(3.5) / np.float32(127),
                              np.float32(0.875) / np.float32(127), 0.0]
    s4 = channel_scales(k, 7)
    assert s4[1].tolist() == [1.0, 0.5, 0.125, 0.0]
