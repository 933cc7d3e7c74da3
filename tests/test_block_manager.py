"""Host bookkeeping of the block pool (CPU): copy-on-write fork and append, reference
counts, swap, stats; and an end-to-end run of the bookkeeping against the oracle's
slot scatter and block copies, checking every sequence's gathered tokens."""
import numpy as np
import pytest

import oracle
from attention_paged_prefix_amd.block_manager import BlockManager, OutOfBlocks


def test_fork_shares_blocks_and_append_copies_on_write():
    m = BlockManager(16)
    t = m.allocate("a", 40)                          # 3 blocks, the last one 8/16 full
    assert t == [0, 1, 2] and m.num_tokens("a") == 40
    m.fork("a", "b")
    assert m.block_table("b") == t and all(m.refcount(x) == 2 for x in t)
    slot, copy = m.append_slot("b")                  # lands in shared block 2 -> private copy
    assert copy == (2, 3) and slot == 3 * 16 + 8
    assert m.block_table("b") == [0, 1, 3] and m.refcount(2) == 1 and m.refcount(3) == 1
    slot, copy = m.append_slot("b")                  # now private: no copy
    assert copy is None and slot == 3 * 16 + 9
    slot, copy = m.append_slot("a")                  # block 2 is a's alone again
    assert copy is None and slot == 2 * 16 + 8
    s = m.stats()
    assert s["used_blocks"] == 4 and s["shared_blocks"] == 2 and s["free_blocks"] == 12


def test_stats_match_the_pages_pool_example():
    """kvboost 0.6.0, "CPU paged attention": a pool of 8192 16-token blocks with 1024 of
    them in use reports a block utilisation of 0.12 (printed to two places; 1024/8192 is
    0.125), 7168 free blocks and 1024 used ones."""
    m = BlockManager(8192)
    m.allocate("prompt", 2048 * 16)                  # 2048 blocks, then fork: shared, not new
    m.fork("prompt", "request")
    m.free("prompt")
    m.free("request")
    for i in range(8):
        m.allocate(i, 128 * 16)                      # 8 x 128 blocks
    s = m.stats()
    assert s["used_blocks"] == 1024
    assert s["free_blocks"] == 7168
    assert s["block_utilization"] == 0.125 and round(s["block_utilization"], 2) == 0.12


def test_append_at_block_boundary_takes_a_new_block():
    m = BlockManager(4)
    m.allocate("a", 32)
    m.fork("a", "b")
    slot, copy = m.append_slot("b")                  # position 32: fresh block, nothing to copy
    assert copy is None and slot == 2 * 16 and m.block_table("b") == [0, 1, 2]
    assert m.refcount(0) == 2 and m.refcount(2) == 1


def test_free_returns_blocks_when_last_reference_goes():
    m = BlockManager(8)
    m.allocate("a", 20)
    m.fork("a", "b")
    m.free("a")
    assert m.stats()["free_blocks"] == 6 and m.refcount(0) == 1
    m.free("b")
    assert m.stats()["free_blocks"] == 8 and m.stats()["used_blocks"] == 0


def test_out_of_blocks():
    m = BlockManager(2)
    m.allocate("a", 32)
    with pytest.raises(OutOfBlocks):
        m.append_slot("a")
    with pytest.raises(OutOfBlocks):
        m.allocate("b", 1)


def test_swap_out_and_in():
    m = BlockManager(6, num_cpu_blocks=4)
    m.allocate("a", 30)
    m.fork("a", "b")
    out = m.swap_out("b")
    assert out == [(0, 0), (1, 1)]
    assert m.refcount(0) == 1 and m.stats()["swapped_sequences"] == 1
    assert m.stats()["cpu_free_blocks"] == 2
    back = m.swap_in("b")
    assert [c for c, _ in back] == [0, 1] and m.stats()["cpu_free_blocks"] == 4
    assert m.block_table("b") == [g for _, g in back] and m.num_tokens("b") == 30


class _OracleBackend:
    def __init__(self, nb, ncpu, shape):
        self.pools = {"gpu": [np.zeros((nb,) + shape, np.uint16), np.zeros((nb,) + shape, np.uint16)],
                      "cpu": [np.zeros((ncpu,) + shape, np.uint16), np.zeros((ncpu,) + shape, np.uint16)]}

    def write(self, slots, kr, vr):
        g = self.pools["gpu"]
        g[0], g[1] = oracle.write_kv(g[0], g[1], kr, vr, np.asarray(slots, np.int64))

    def copy(self, src, dst, s_ids, d_ids):
        a, b = self.pools[src], self.pools[dst]
        b[0], b[1] = oracle.copy_blocks(a[0], a[1], b[0], b[1], s_ids, d_ids)


def test_random_script_keeps_every_sequence_intact():
    import blockscript
    nb, ncpu = 48, 24
    be = _OracleBackend(nb, ncpu, (2, 16, 8))
    m, expect = blockscript.run(be, nb, ncpu, 400, 11, (2, 8))
    assert expect
    # bring every swapped sequence back (space permitting), then check every sequence
    for sq in list(m._swapped):
        try:
            pairs = m.swap_in(sq)
        except OutOfBlocks:
            continue
        be.copy("cpu", "gpu", [c for c, _ in pairs], [g for _, g in pairs])
    checked = 0
    for sq, (ks, vs) in expect.items():
        if sq in m._swapped:
            continue
        n = m.num_tokens(sq)
        assert n == len(ks)
        table = np.asarray(m.block_table(sq), np.int32)
        assert np.array_equal(oracle.gather_kv(be.pools["gpu"][0], table, n), np.stack(ks))
        assert np.array_equal(oracle.gather_kv(be.pools["gpu"][1], table, n), np.stack(vs))
        checked += 1
    assert checked >= 3
    s = m.stats()
    assert s["used_blocks"] + s["free_blocks"] == nb
