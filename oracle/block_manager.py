"""Block manager and contiguous reservation — test infrastructure only.

A plain statement of the bookkeeping that decides which physical blocks a
sequence owns, written from "PagedAttention" (shubhamtatvamasi.com):

* section "The idea: page the KV cache": blocks come one at a time from a
  free list, and a sequence takes a new one only when its last block is full,
  so it wastes at most one partially filled block;
* section "Sharing and copy-on-write" and the FAQ entry on copy-on-write for
  parallel sampling: a block's reference count is the number of sequences
  whose table holds it; forking a sequence shares all its blocks; a sequence
  about to write into a shared, partially filled block first takes a new
  block, copies the existing tokens into it, drops its reference to the old
  block and writes into the copy; full blocks are never written again;
* the introduction and its five-request animation: the contiguous baseline
  reserves a request's maximum length up front, and free space splits into
  gaps.

Readings (the pages are silent on order): the free list is a stack that
starts with blocks num_blocks-1 .. 0 pushed in that order (the first blocks
handed out are 0, 1, 2, ...); freeing a sequence pushes its blocks whose
count reaches zero in logical-block order.  A batch of appends is applied in
the listed order and fails as a whole if the free list cannot cover it.  The
contiguous allocator places a reservation at the lowest-addressed gap that
fits.

The code mirrors nothing from the library: lists and dicts, one token at a
time.
"""


class OutOfBlocks(Exception):
    pass


class BlockManager:
    def __init__(self, num_blocks, block_size, max_blocks_per_seq):
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = list(range(num_blocks - 1, -1, -1))  # pop() gives 0 first
        self.refs = [0] * num_blocks
        self.tokens_in = [0] * num_blocks  # token slots written per block
        self.tables = {}                   # seq -> list of physical blocks
        self.lengths = {}                  # seq -> tokens

    # -- allocation ------------------------------------------------------
    def _available(self):
        return len(self.free)

    def _take(self):
        if not self.free:
            raise OutOfBlocks()
        b = self.free.pop()
        self.refs[b] = 1
        self.tokens_in[b] = 0
        return b

    def _release(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free.append(b)

    # -- operations ------------------------------------------------------
    def add_sequence(self, seq, num_tokens):
        """A prompt of num_tokens tokens; returns the slot of each token."""
        assert seq not in self.tables
        nblocks = -(-num_tokens // self.block_size)
        assert nblocks <= self.max_blocks_per_seq
        if nblocks > self._available():
            raise OutOfBlocks()
        table = []
        for i in range(nblocks):
            b = self._take()
            self.tokens_in[b] = min(self.block_size,
                                    num_tokens - i * self.block_size)
            table.append(b)
        self.tables[seq] = table
        self.lengths[seq] = num_tokens
        return [table[t // self.block_size] * self.block_size
                + t % self.block_size for t in range(num_tokens)]

    def fork(self, parent, child):
        assert parent in self.tables and child not in self.tables
        self.tables[child] = list(self.tables[parent])
        for b in self.tables[child]:
            self.refs[b] += 1
        self.lengths[child] = self.lengths[parent]

    def _append_one(self, seq, pairs, counts):
        table = self.tables[seq]
        n = self.lengths[seq]
        offset = n % self.block_size
        if offset == 0:                       # no block yet, or last one full
            assert len(table) < self.max_blocks_per_seq
            table.append(self._take())
        elif self.refs[table[-1]] > 1:        # shared, partially filled
            old = table[-1]
            new = self._take()
            self.tokens_in[new] = self.tokens_in[old]  # the copied tokens
            counts.append(self.tokens_in[old])
            self._release(old)
            table[-1] = new
            pairs.append((old, new))
        b = table[-1]
        self.tokens_in[b] += 1
        self.lengths[seq] = n + 1
        return b * self.block_size + offset

    def append(self, seqs, with_counts=False):
        """One new token for each sequence, in order.  Returns (slots,
        copy pairs) and, with_counts, the tokens each copy carries (those the
        old block holds); raises OutOfBlocks (and changes nothing) if the
        free list runs out part way."""
        assert len(set(seqs)) == len(seqs)
        saved = self._snapshot()
        pairs, counts = [], []
        try:
            slots = [self._append_one(s, pairs, counts) for s in seqs]
        except OutOfBlocks:
            self._restore(saved)
            raise
        if with_counts:
            return slots, pairs, counts
        return slots, pairs

    def _snapshot(self):
        return (list(self.free), list(self.refs), list(self.tokens_in),
                {s: list(t) for s, t in self.tables.items()},
                dict(self.lengths))

    def _restore(self, saved):
        (self.free, self.refs, self.tokens_in, self.tables,
         self.lengths) = saved

    def free_sequence(self, seq):
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lengths[seq]

    # -- views -----------------------------------------------------------
    def table(self, seq):
        return list(self.tables[seq])

    def stats(self):
        used = [b for b, r in enumerate(self.refs) if r > 0]
        stored = sum(self.tokens_in[b] for b in used)
        return {
            "free_blocks": self._available(),
            "used_blocks": len(used),
            "shared_blocks": sum(1 for b in used if self.refs[b] > 1),
            "live_sequences": len(self.tables),
            "logical_tokens": sum(self.lengths.values()),
            "stored_tokens": stored,
            "wasted_slots": len(used) * self.block_size - stored,
        }


class PrefixCachingBlockManager(BlockManager):
    """The manager with prompt-prefix caching ("PagedAttention",
    shubhamtatvamasi.com, "Sharing and copy-on-write": different requests
    with the same system prompt share blocks; "Choosing the block size":
    sharing goes by whole blocks).

    Readings: a full block filled from a prompt is registered under the
    prompt's tokens up to and including that block; a later prompt takes the
    registered blocks of its leading full blocks, in order, until the first
    one that is not registered (and registers its new full blocks, as long
    as their prefix is not registered already); partially filled blocks are
    never shared this way; a registered block with no reference left stays
    registered on an evictable list (oldest release first) and is reused --
    losing its registration -- only when no plain free block is left; blocks
    filled by appends carry no token ids and are not registered.  Written
    with the whole prefix as the key (a tuple of token ids), so there is no
    hashing here at all.
    """

    def __init__(self, num_blocks, block_size, max_blocks_per_seq):
        super().__init__(num_blocks, block_size, max_blocks_per_seq)
        self.registry = {}     # prefix tuple -> block
        self.key_of = {}       # block -> prefix tuple
        self.evictable = []    # oldest release first
        self.hit_blocks = 0

    def _available(self):
        return len(self.free) + len(self.evictable)

    def _take(self):
        if self.free:
            return super()._take()
        if not self.evictable:
            raise OutOfBlocks()
        b = self.evictable.pop(0)
        del self.registry[self.key_of.pop(b)]
        self.refs[b] = 1
        self.tokens_in[b] = 0
        return b

    def _release(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            if b in self.key_of:
                self.evictable.append(b)
            else:
                self.free.append(b)

    def add_sequence_tokens(self, seq, tokens):
        """Returns (slots of every token, tokens whose blocks were cached)."""
        assert seq not in self.tables
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        n = len(tokens)
        nblocks = -(-n // bs)
        assert nblocks <= self.max_blocks_per_seq
        hits = []
        for i in range(n // bs):
            b = self.registry.get(tuple(tokens[:(i + 1) * bs]))
            if b is None:
                break
            hits.append(b)
        revived = sum(1 for b in hits if self.refs[b] == 0)
        if nblocks - len(hits) > self._available() - revived:
            raise OutOfBlocks()
        table = []
        for b in hits:
            if self.refs[b] == 0:
                self.evictable.remove(b)
            self.refs[b] += 1
            table.append(b)
        self.hit_blocks += len(hits)
        registering = True
        for i in range(len(hits), nblocks):
            b = self._take()
            self.tokens_in[b] = min(bs, n - i * bs)
            if registering and n - i * bs >= bs:
                key = tuple(tokens[:(i + 1) * bs])
                if key in self.registry:
                    registering = False
                else:
                    self.registry[key] = b
                    self.key_of[b] = key
            table.append(b)
        self.tables[seq] = table
        self.lengths[seq] = n
        slots = [table[t // bs] * bs + t % bs for t in range(n)]
        return slots, len(hits) * bs

    def _snapshot(self):
        return (super()._snapshot(), dict(self.registry), dict(self.key_of),
                list(self.evictable))

    def _restore(self, saved):
        base, self.registry, self.key_of, self.evictable = saved
        super()._restore(base)

    def prefix_stats(self):
        return {"registered": len(self.key_of),
                "evictable": len(self.evictable),
                "hit_blocks": self.hit_blocks}


class ContiguousAllocator:
    """Max-length reservations in one buffer of token slots, first fit."""

    def __init__(self, num_slots):
        self.num_slots = num_slots
        self.owned = {}  # request -> (start, length)

    def gaps(self):
        spans = sorted(self.owned.values())
        out, pos = [], 0
        for start, length in spans:
            if start > pos:
                out.append((pos, start - pos))
            pos = start + length
        if pos < self.num_slots:
            out.append((pos, self.num_slots - pos))
        return out

    def reserve(self, req, num_slots):
        """Start slot of the reservation, or None when no gap fits."""
        assert req not in self.owned
        for start, length in self.gaps():
            if length >= num_slots:
                self.owned[req] = (start, num_slots)
                return start
        return None

    def release(self, req):
        del self.owned[req]

    def stats(self):
        g = self.gaps()
        free = sum(length for _, length in g)
        return {"free_slots": free,
                "largest_gap": max((length for _, length in g), default=0),
                "reserved_slots": self.num_slots - free}
