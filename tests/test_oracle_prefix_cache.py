"""Pins for the oracle's prompt-prefix cache (CPU only).

What fixes it, other than itself:

* the pages' statement ("PagedAttention", "Sharing and copy-on-write"):
  requests with the same system prompt share blocks -- checked on prompts
  built around one system prompt, block by block;
* whole-block granularity ("Choosing the block size": sharing goes by
  blocks): the tail of a shared prefix that does not fill a block is not
  shared;
* a direct count: for any two prompts added while nothing is evicted, the
  number of blocks they share is the number of leading full blocks on which
  the two token lists agree, computed by comparing the lists;
* invariants over random operations: a block's reference count equals the
  tables holding it; the free list, the evictable list and the referenced
  blocks partition the pool; every registered block is full and holds the
  prefix it is registered under.
"""

import numpy as np
import pytest

from oracle.block_manager import OutOfBlocks, PrefixCachingBlockManager as PC


def shared_leading_blocks(p1, p2, bs):
    k = 0
    while (k + 1) * bs <= min(len(p1), len(p2)) and \
            p1[:(k + 1) * bs] == p2[:(k + 1) * bs]:
        k += 1
    return k


def test_same_system_prompt_shares_its_full_blocks():
    bs = 4
    system = list(range(100, 110))                   # 10 tokens: 2.5 blocks
    pc = PC(32, bs, 16)
    s1, c1 = pc.add_sequence_tokens(0, system + [1, 2, 3])
    s2, c2 = pc.add_sequence_tokens(1, system + [7, 8, 9, 10, 11])
    assert c1 == 0 and c2 == 8                        # two full blocks cached
    t1, t2 = pc.table(0), pc.table(1)
    assert t1[:2] == t2[:2] and t1[2] != t2[2]        # partial block private
    assert [pc.refs[b] for b in t1[:2]] == [2, 2]
    assert s2[:8] == s1[:8]                           # same slots, same K/V
    assert pc.prefix_stats()["hit_blocks"] == 2


def test_identical_prompts_share_everything_full():
    bs = 4
    pc = PC(16, bs, 8)
    p = list(range(12))
    pc.add_sequence_tokens(0, p)
    _, cached = pc.add_sequence_tokens(1, p)
    assert cached == 12 and pc.table(0) == pc.table(1)
    st = pc.stats()
    assert st["used_blocks"] == 3 and st["shared_blocks"] == 3


def test_a_different_token_stops_sharing_at_its_block():
    bs = 4
    pc = PC(16, bs, 8)
    p = list(range(12))
    q = p.copy()
    q[5] = 99                                         # in block 1
    pc.add_sequence_tokens(0, p)
    _, cached = pc.add_sequence_tokens(1, q)
    assert cached == 4
    assert pc.table(0)[0] == pc.table(1)[0]
    assert pc.table(0)[1] != pc.table(1)[1]


def test_released_prefix_is_reused_and_evicted_last():
    bs = 4
    pc = PC(6, bs, 6)
    a = [1] * 8 + [2] * 3                             # 2 full + partial
    pc.add_sequence_tokens(0, a)
    blocks_a = pc.table(0)
    pc.free_sequence(0)
    st = pc.prefix_stats()
    assert st["registered"] == 2 and st["evictable"] == 2
    assert pc.stats()["free_blocks"] == 6
    # the same prefix comes back from the evictable list
    _, cached = pc.add_sequence_tokens(1, a[:8] + [5])
    assert cached == 8 and pc.table(1)[:2] == blocks_a[:2]
    pc.free_sequence(1)
    # exhaust the plain free blocks: the oldest released cached block goes
    b = [9] * 16                                      # 4 new full blocks
    pc.add_sequence_tokens(2, b)
    assert pc.prefix_stats()["evictable"] == 2        # still cached
    c = [8] * 8                                       # needs 2: evicts both
    pc.add_sequence_tokens(3, c)
    assert pc.prefix_stats()["evictable"] == 0
    pc.free_sequence(3)
    _, cached = pc.add_sequence_tokens(4, a[:8])      # (evicts c's blocks)
    assert cached == 0                                # prefix was evicted


def test_all_or_nothing_when_blocks_run_out():
    pc = PC(3, 4, 8)
    pc.add_sequence_tokens(0, list(range(8)))
    with pytest.raises(OutOfBlocks):
        pc.add_sequence_tokens(1, list(range(100, 112)))
    assert 1 not in pc.tables and pc.stats()["free_blocks"] == 1
    # a hit needs no new block: fits although only one block is free
    _, cached = pc.add_sequence_tokens(1, list(range(8)) + [42])
    assert cached == 8


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sharing_count_matches_direct_comparison(seed):
    rng = np.random.default_rng(seed)
    bs = 4
    systems = [list(rng.integers(0, 50, 11)) for _ in range(3)]
    prompts = []
    for i in range(12):
        s = systems[i % 3]
        cut = int(rng.integers(0, len(s) + 1))
        prompts.append([int(t) for t in s[:cut]] +
                       [int(t) for t in rng.integers(0, 50, int(rng.integers(0, 9)))])
    pc = PC(400, bs, 64)                              # nothing is evicted
    for i, p in enumerate(prompts):
        pc.add_sequence_tokens(i, p)
    for i in range(len(prompts)):
        for j in range(i):
            k = shared_leading_blocks(prompts[i], prompts[j], bs)
            ti, tj = pc.table(i), pc.table(j)
            n_same = 0
            while n_same < min(len(ti), len(tj)) and ti[n_same] == tj[n_same]:
                n_same += 1
            assert n_same == k, (i, j)


def check_invariants(pc, nblocks):
    holders = [0] * nblocks
    for t in pc.tables.values():
        for b in t:
            holders[b] += 1
    assert holders == pc.refs
    free, evict = set(pc.free), set(pc.evictable)
    used = {b for b in range(nblocks) if pc.refs[b] > 0}
    assert len(free) == len(pc.free) and len(evict) == len(pc.evictable)
    assert free | evict | used == set(range(nblocks))
    assert not (free & evict) and not (free & used) and not (evict & used)
    for key, b in pc.registry.items():
        assert pc.key_of[b] == key
        assert pc.tokens_in[b] == pc.block_size
        assert len(key) % pc.block_size == 0
    assert evict <= set(pc.key_of)


@pytest.mark.parametrize("seed", [3, 4])
def test_invariants_under_random_operations(seed):
    rng = np.random.default_rng(seed)
    nblocks, bs = 24, 4
    pc = PC(nblocks, bs, 12)
    systems = [list(rng.integers(0, 9, 9)) for _ in range(2)]
    live = set()
    for step in range(600):
        op = int(rng.integers(0, 10))
        idle = [s for s in range(16) if s not in live]
        if op < 3 and idle:
            s = int(rng.choice(idle))
            sys = systems[int(rng.integers(0, 2))]
            p = [int(t) for t in sys[:int(rng.integers(0, 10))]] + \
                [int(t) for t in rng.integers(0, 9, int(rng.integers(0, 6)))]
            try:
                pc.add_sequence_tokens(s, p)
                live.add(s)
            except OutOfBlocks:
                pass
        elif op < 4 and live and idle:
            p, c = int(rng.choice(sorted(live))), int(rng.choice(idle))
            pc.fork(p, c)
            live.add(c)
        elif op < 7 and live:
            seqs = [int(x) for x in rng.choice(sorted(live),
                                               int(rng.integers(1, len(live) + 1)),
                                               replace=False)]
            try:
                pc.append(seqs)
            except OutOfBlocks:
                pass
        elif live:
            s = int(rng.choice(sorted(live)))
            pc.free_sequence(s)
            live.discard(s)
        check_invariants(pc, nblocks)
