"""Pins of the block-manager oracle (CPU) against what the pages fix.

"PagedAttention" (shubhamtatvamasi.com): the worked example's block count
and tail waste ("How attention reads paged memory", block size 4, 22
tokens), the five-request animation and the at-most-one-partial-block rule
("The idea: page the KV cache"), the 8K/300-token reservation waste and the
gaps of external fragmentation (introduction), and the copy-on-write steps of
the FAQ entry on parallel sampling ("Sharing and copy-on-write").  Invariants
that hold for any sequence of operations are checked on random runs."""

import numpy as np
import pytest

from oracle.block_manager import BlockManager, ContiguousAllocator, OutOfBlocks


def test_worked_example_block_count_and_tail():
    bm = BlockManager(num_blocks=16, block_size=4, max_blocks_per_seq=8)
    slots = bm.add_sequence(0, 22)
    table = bm.table(0)
    assert len(table) == 6                     # ceil(22 / 4)
    assert slots == [table[t // 4] * 4 + t % 4 for t in range(22)]
    st = bm.stats()
    assert st["used_blocks"] == 6 and st["free_blocks"] == 10
    assert st["wasted_slots"] == 2             # the last block holds 2 of 4


def test_reservation_waste_closed_form():
    # an 8K reservation answered in 300 tokens leaves > 96 % unused
    ca = ContiguousAllocator(8192)
    assert ca.reserve(0, 8192) == 0
    unused = 1 - 300 / ca.stats()["reserved_slots"]
    assert unused > 0.96
    assert unused == pytest.approx(1 - 300 / 8192)


def test_five_requests_animation():
    lengths = [7, 12, 5, 9, 10]
    ca = ContiguousAllocator(64)
    starts = [ca.reserve(i, 20) for i in range(5)]
    assert starts == [0, 20, 40, None, None]   # D and E wait
    assert ca.stats()["free_slots"] == 4
    bm = BlockManager(num_blocks=16, block_size=4, max_blocks_per_seq=16)
    for i in range(5):
        bm.add_sequence(i, 0)
    for step in range(max(lengths)):
        bm.append([i for i, L in enumerate(lengths) if L > step])
    for i, L in enumerate(lengths):
        assert bm.lengths[i] == L
        assert len(bm.table(i)) * 4 - L < 4    # at most one partial block
    assert bm.stats()["used_blocks"] == sum(-(-L // 4) for L in lengths)


def test_external_fragmentation():
    ca = ContiguousAllocator(64)
    for i in range(3):
        ca.reserve(i, 20)
    ca.release(1)
    st = ca.stats()
    assert st["free_slots"] == 24 and st["largest_gap"] == 20
    assert ca.reserve(3, 21) is None           # enough in total, no gap fits
    assert ca.reserve(4, 20) == 20


def test_copy_on_write_steps_for_parallel_sampling():
    bm = BlockManager(num_blocks=32, block_size=4, max_blocks_per_seq=8)
    bm.add_sequence(0, 10)                     # 2 full blocks + 2 of 4
    full0, full1, partial = bm.table(0)
    for child in (1, 2, 3):
        bm.fork(0, child)
    assert [bm.refs[b] for b in (full0, full1, partial)] == [4, 4, 4]
    # the first sample to append copies the shared partial block
    slots, pairs = bm.append([1])
    (old, new), = pairs
    assert old == partial and new not in (full0, full1, partial)
    assert bm.table(1) == [full0, full1, new]
    assert bm.refs[partial] == 3 and bm.refs[new] == 1
    assert bm.tokens_in[new] == 3              # 2 copied + the new token
    assert slots == [new * 4 + 2]
    # full blocks stay shared
    assert bm.refs[full0] == 4 and bm.refs[full1] == 4
    # the next two copy as well; the last sharer writes in place
    _, p2 = bm.append([2])
    _, p3 = bm.append([3])
    assert len(p2) == 1 and len(p3) == 1
    assert bm.refs[partial] == 1
    slots, p0 = bm.append([0])
    assert p0 == [] and slots == [partial * 4 + 2]
    # a sequence copies at most once: its block is now its own
    _, again = bm.append([1, 2, 3, 0])
    assert again == []


def test_full_shared_block_is_never_copied():
    bm = BlockManager(num_blocks=8, block_size=4, max_blocks_per_seq=8)
    bm.add_sequence(0, 8)                      # two full blocks
    bm.fork(0, 1)
    _, pairs = bm.append([1])
    assert pairs == []
    assert len(bm.table(1)) == 3 and bm.table(1)[:2] == bm.table(0)
    assert all(bm.refs[b] == 2 for b in bm.table(0))


def test_batch_copy_counts_follow_the_order():
    # siblings in one batch: all but the last sharer copy
    bm = BlockManager(num_blocks=16, block_size=4, max_blocks_per_seq=8)
    bm.add_sequence(0, 6)
    bm.fork(0, 1)
    bm.fork(0, 2)
    _, pairs = bm.append([2, 0, 1])
    assert len(pairs) == 2
    assert [src for src, _ in pairs] == [bm.table(1)[-1]] * 2  # 1 kept it
    last = [bm.table(s)[-1] for s in (0, 1, 2)]
    assert len(set(last)) == 3


def test_out_of_blocks_changes_nothing():
    bm = BlockManager(num_blocks=3, block_size=4, max_blocks_per_seq=4)
    bm.add_sequence(0, 4)
    bm.add_sequence(1, 4)
    bm.add_sequence(2, 3)
    before = (list(bm.free), list(bm.refs), {s: bm.table(s) for s in bm.tables})
    with pytest.raises(OutOfBlocks):
        bm.append([2, 0])                      # 2 fits in place, 0 needs one
    assert (list(bm.free), list(bm.refs),
            {s: bm.table(s) for s in bm.tables}) == before
    with pytest.raises(OutOfBlocks):
        bm.add_sequence(3, 1)


def test_freed_blocks_come_back_last_freed_first():
    bm = BlockManager(num_blocks=8, block_size=2, max_blocks_per_seq=8)
    bm.add_sequence(0, 5)                      # blocks 0, 1, 2
    bm.add_sequence(1, 2)                      # block 3
    assert bm.table(0) == [0, 1, 2] and bm.table(1) == [3]
    bm.free_sequence(0)
    bm.add_sequence(2, 6)
    assert bm.table(2) == [2, 1, 0]


def _check_invariants(bm, nblocks):
    holders = [0] * nblocks
    for seq, table in bm.tables.items():
        assert len(set(table)) == len(table)
        L = bm.lengths[seq]
        assert len(table) == -(-L // bm.block_size)
        for i, b in enumerate(table):
            holders[b] += 1
            assert bm.tokens_in[b] == min(bm.block_size, L - i * bm.block_size)
    assert holders == bm.refs
    free = set(bm.free)
    assert len(free) == len(bm.free)
    assert free == {b for b in range(nblocks) if holders[b] == 0}


def test_random_operations_keep_the_invariants():
    rng = np.random.default_rng(7)
    nblocks, bs = 64, 4
    bm = BlockManager(nblocks, bs, max_blocks_per_seq=64)
    live = set()
    for step in range(600):
        op = rng.integers(0, 10)
        free_ids = [s for s in range(24) if s not in live]
        try:
            if op < 2 and free_ids:
                s = int(rng.choice(free_ids))
                bm.add_sequence(s, int(rng.integers(0, 13)))
                live.add(s)
            elif op < 4 and live and free_ids:
                p = int(rng.choice(sorted(live)))
                c = int(rng.choice(free_ids))
                bm.fork(p, c)
                live.add(c)
            elif op < 8 and live:
                k = int(rng.integers(1, len(live) + 1))
                seqs = [int(x) for x in rng.choice(sorted(live), k, replace=False)]
                bm.append(seqs)
            elif live:
                s = int(rng.choice(sorted(live)))
                bm.free_sequence(s)
                live.discard(s)
        except OutOfBlocks:
            pass
        _check_invariants(bm, nblocks)
