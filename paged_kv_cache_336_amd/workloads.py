"""Seeded synthetic decode-step workloads (inputs only; no attention arithmetic).

This module builds the inputs of one decode step of a single attention layer:
a paged K/V pool, per-sequence block tables and lengths, query rows, the new
key/value rows with their slot mapping, and copy-on-write block pairs.  It is
the one module that both the CPU oracle and the HIP path are fed from; it
computes none of the method's results (no attention, no cache write, no block
copy).  What it does compute is the host-side bookkeeping a block manager
would do: which physical block each logical block lives in, where each new
token goes, and which shared block must be duplicated before an append.

Terminology and structure follow "PagedAttention" (shubhamtatvamasi.com):
fixed-size blocks handed out from a free list ("The idea: page the KV cache"),
a block table per sequence ("How attention reads paged memory"), and
copy-on-write of a shared, partially filled last block, at most one per
sequence ("Sharing and copy-on-write").

Storage conventions: ``"f32"`` float32, ``"f16"`` float16, ``"bf16"`` uint16
bfloat16 bits, ``"fp8_e4m3"`` / ``"fp8_e5m2"`` uint8 OCP E4M3 / E5M2 codes.  Slots that hold no live
token are poisoned with NaN (0x7F for fp8) so that a stray read shows up in
the output instead of passing silently.

Value recipe: every live value is float32 N(0, 1) cast to the storage type
with round-to-nearest-even.  Random draws come from
``numpy.random.default_rng([336, k])`` for workload family k, in the order
lengths -> block-id permutation -> K pool -> V pool -> Q -> new K -> new V;
each pool takes one integer from that stream as the key of its own chunked
streams (so large pools are drawn on several threads).
"""

from dataclasses import dataclass, field, replace
import math

import numpy as np

SEED_BASE = 336
KINDS = ("f32", "f16", "bf16", "fp8_e4m3", "fp8_e5m2")
FP8_KINDS = ("fp8_e4m3", "fp8_e5m2")
_NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16,
               "fp8_e4m3": np.uint8, "fp8_e5m2": np.uint8}
_FP8_LIMIT = {"fp8_e4m3": 448.0, "fp8_e5m2": 57344.0}


# ----------------------------------------------------------------------------
# value synthesis
# ----------------------------------------------------------------------------

def _cast_from_f32(x, kind):
    """float32 array -> storage array (RNE); fp8 handled separately."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if kind == "f32":
        return x
    if kind == "f16":
        return x.astype(np.float16)
    if kind == "bf16":
        import torch
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(kind)


def _fp8_codes_from_f32(x, scale, kind="fp8_e4m3"):
    """Pool contents of an fp8 cache [.., Hkv, D]: codes of x/scale via
    torch's float8 cast (library routine), clamped into the finite range
    first; scale is one value or one per kv head."""
    import torch
    lim = _FP8_LIMIT[kind]
    y = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    s = np.asarray(scale, dtype=np.float32)
    if s.ndim == 3:                        # per token: [nb, bs, Hkv]
        s = torch.from_numpy(np.ascontiguousarray(s)[..., None])
    else:
        s = torch.from_numpy(s.reshape(-1))
        if s.numel() > 1:
            s = s.reshape(s.numel(), 1)    # broadcast over [.., Hkv, D]
    y = (y / s).clamp_(-lim, lim)
    dt = torch.float8_e4m3fn if kind == "fp8_e4m3" else torch.float8_e5m2
    return y.to(dt).view(torch.uint8).numpy()


def poison_value(kind):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan),
            "bf16": np.uint16(0x7FC0), "fp8_e4m3": np.uint8(0x7F),
            "fp8_e5m2": np.uint8(0x7F)}[kind]


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


# ----------------------------------------------------------------------------
# the workload record
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    """One decode step's inputs.  Pools hold the state *before* the step:
    slots of the tokens written this step and copy-on-write destinations are
    poisoned, like every other slot that holds no live token."""
    name: str
    q_kind: str
    kv_kind: str
    src_kind: str            # dtype of the new key/value rows
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float             # softmax scale, a float32 value
    query: np.ndarray        # [S, Hq, D]
    k_pool: np.ndarray       # [nb, bs, Hkv, D]
    v_pool: np.ndarray
    block_tables: np.ndarray  # int32 [S, max_blocks]
    seq_lens: np.ndarray     # int32 [S], including this step's token
    key: np.ndarray          # [T, Hkv, D] new rows (src_kind)
    value: np.ndarray
    slot_mapping: np.ndarray  # int32 [T]
    copy_pairs: np.ndarray   # int32 [P, 2] (src, dst)
    k_scale: float = 1.0     # float32 value(s); fp8 caches: one, per kv head,
                             # or per (slot, kv head) [nb, bs, Hkv]
    v_scale: float = 1.0
    # Extra disjoint copies of (tables, slots, pairs) over the same pool,
    # for rotating benchmark steps through more memory than the caches hold.
    replicas: list = field(default_factory=list)
    note: str = ""

    @property
    def num_seqs(self):
        return int(self.block_tables.shape[0])

    @property
    def num_blocks(self):
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self):
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    @property
    def num_tokens(self):
        return int(self.slot_mapping.shape[0])


# ----------------------------------------------------------------------------
# block-manager bookkeeping (host side)
# ----------------------------------------------------------------------------

def blocks_for(length, block_size):
    """Table entries a sequence of ``length`` tokens needs: ceil(L / bs)."""
    return -(-int(length) // int(block_size))


def slot_of(block_table_row, position, block_size):
    """Flat slot of token ``position``: physical block * bs + offset."""
    return int(block_table_row[position // block_size]) * block_size + \
        position % block_size


def live_slot_mask(num_blocks, block_size, block_tables, cached_lens):
    """Boolean [nb, bs]: slots holding one of positions 0..cached_len-1 of
    some sequence."""
    mask = np.zeros((num_blocks, block_size), dtype=bool)
    for row, n_tok in zip(block_tables, cached_lens):
        n_tok = int(n_tok)
        full, rem = divmod(n_tok, block_size)
        if full:
            mask[np.asarray(row[:full], dtype=np.int64)] = True
        if rem:
            mask[int(row[full]), :rem] = True
    return mask


def _draw_chunks(seed_key, num_blocks, block_size, hkv, d, chunk_blocks):
    """N(0,1) float32 pool values, drawn chunk by chunk from independent
    streams ``default_rng(seed_key + [chunk])`` on a thread pool, so the
    result does not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    x = np.empty((num_blocks, block_size, hkv, d), dtype=np.float32)
    starts = list(range(0, num_blocks, chunk_blocks))

    def work(ci):
        b0 = starts[ci]
        b1 = min(num_blocks, b0 + chunk_blocks)
        g = np.random.default_rng(list(seed_key) + [ci])
        x[b0:b1] = g.standard_normal(size=(b1 - b0, block_size, hkv, d),
                                     dtype=np.float32)
    workers = max(1, min(16, os.cpu_count() or 1, len(starts)))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(work, range(len(starts))))
    return x


def _fill_pool(seed_key, num_blocks, block_size, hkv, d, kind, live,
               chunk_blocks=512, per_head=False, per_token=False):
    """N(0,1) values at live slots, poison elsewhere, in storage kind.

    For an fp8 cache the scale is max|live value| / (largest finite code
    value: 448 for E4M3, 57344 for E5M2) as a float32, per tensor or, with
    per_head, per kv head (float32 [Hkv]); with per_token, each live (slot,
    kv head) row gets its own, that row's max|value| / largest code times a
    factor drawn from [1, 1.5) (so not every row reaches the largest code),
    as float32 [num_blocks, block_size, Hkv] with NaN at slots that hold no
    token; returns (pool, scale), scale 1.0 for other kinds."""
    x = _draw_chunks(seed_key, num_blocks, block_size, hkv, d, chunk_blocks)
    poison = poison_value(kind)
    scale = 1.0
    if kind in FP8_KINDS and per_token:
        lim = np.float32(_FP8_LIMIT[kind])
        amax = np.abs(x).max(axis=3)               # [nb, bs, Hkv]
        widen = np.random.default_rng(list(seed_key) + [9]).uniform(
            1.0, 1.5, size=amax.shape).astype(np.float32)
        scale = np.where(amax > 0, amax / lim * widen,
                         np.float32(1)).astype(np.float32)
        scale[~live] = np.nan
        pool = _fp8_codes_from_f32(x, scale, kind)
        pool[~live] = poison
        return pool, scale
    if kind in FP8_KINDS:
        lim = _FP8_LIMIT[kind]
        sel = np.abs(x[live])                      # [n_live, Hkv, D]
        if per_head:
            amax = sel.max(axis=(0, 2)) if sel.size else np.zeros(hkv)
            scale = np.where(amax > 0, amax / lim, 1.0).astype(np.float32)
        else:
            amax = float(sel.max()) if sel.size else 0.0
            scale = float(np.float32(amax / lim)) if amax > 0 else 1.0
        del sel
        pool = _fp8_codes_from_f32(x, scale, kind)
    else:
        pool = _cast_from_f32(x, kind)
    del x
    pool[~live] = poison
    return pool, scale


def _unused_column_fill(block_tables, counts, filler):
    for i, n in enumerate(counts):
        block_tables[i, n:] = filler


# ----------------------------------------------------------------------------
# generic single-step builder
# ----------------------------------------------------------------------------

def _build(name, rng, *, q_kind, kv_kind, src_kind, hq, hkv, d, bs, nb,
           block_tables, seq_lens, cached_lens, slot_mapping, copy_pairs,
           replicas=(), note="", live_extra=None, per_head_scales=False,
           per_token_scales=False):
    """Draw pool values and rows for an already-laid-out step."""
    live = live_slot_mask(nb, bs, block_tables, cached_lens)
    for rep in replicas:
        live |= live_slot_mask(nb, bs, rep["block_tables"], cached_lens)
    if live_extra is not None:
        live |= live_extra
    S = block_tables.shape[0]
    T = len(slot_mapping)
    key_base = [int(v) for v in rng.integers(0, 2**31, size=2)]
    k_pool, k_scale = _fill_pool([SEED_BASE, key_base[0], 0], nb, bs, hkv, d,
                                 kv_kind, live, per_head=per_head_scales,
                                 per_token=per_token_scales)
    v_pool, v_scale = _fill_pool([SEED_BASE, key_base[1], 1], nb, bs, hkv, d,
                                 kv_kind, live, per_head=per_head_scales,
                                 per_token=per_token_scales)
    query = _cast_from_f32(_normal(rng, (S, hq, d)), q_kind)
    key = _cast_from_f32(_normal(rng, (T, hkv, d)), src_kind)
    value = _cast_from_f32(_normal(rng, (T, hkv, d)), src_kind)
    return Workload(
        name=name, q_kind=q_kind, kv_kind=kv_kind, src_kind=src_kind,
        num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
        scale=float(np.float32(1.0 / math.sqrt(d))),
        query=query, k_pool=k_pool, v_pool=v_pool,
        block_tables=np.ascontiguousarray(block_tables, dtype=np.int32),
        seq_lens=np.asarray(seq_lens, dtype=np.int32),
        key=key, value=value,
        slot_mapping=np.asarray(slot_mapping, dtype=np.int32),
        copy_pairs=np.asarray(copy_pairs, dtype=np.int32).reshape(-1, 2),
        k_scale=k_scale, v_scale=v_scale,
        replicas=list(replicas), note=note)


def _decode_layout(lens, bs, ids, max_blocks, filler):
    """Tables for sequences of ``lens`` tokens (after the append), taking
    physical ids in order from ``ids``; one new token per sequence at
    position L-1."""
    S = len(lens)
    counts = [blocks_for(L, bs) for L in lens]
    tables = np.zeros((S, max_blocks), dtype=np.int32)
    pos = 0
    for i, n in enumerate(counts):
        tables[i, :n] = ids[pos:pos + n]
        pos += n
    _unused_column_fill(tables, counts, filler)
    slots = [slot_of(tables[i], int(L) - 1, bs) for i, L in enumerate(lens)]
    return tables, np.asarray(slots, dtype=np.int32), pos


def lognormal_lengths(rng, n, median, cap, sigma=1.0):
    """L = clamp(round(exp(ln(median) + sigma * Z)), 1, cap)."""
    z = rng.standard_normal(n)
    L = np.rint(np.exp(math.log(median) + sigma * z))
    return np.clip(L, 1, cap).astype(np.int64)


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------

WORKED_EXAMPLE_BLOCKS = (7, 2, 11, 5, 9, 0)


def worked_example(seed_family=0):
    """One sequence of 22 tokens, block size 4, on physical blocks
    7, 2, 11, 5, 9, 0 of a 16-block pool ("PagedAttention",
    shubhamtatvamasi.com, figure in "How attention reads paged memory");
    fp32, 1 query head, 1 cache head, head_dim 64.  All 22 tokens are
    written this step through the slot mapping block_id*4 + offset; blocks
    outside the table hold either other requests' rows or poison."""
    rng = np.random.default_rng([SEED_BASE, seed_family])
    bs, nb, L, d = 4, 16, 22, 64
    table = np.asarray([WORKED_EXAMPLE_BLOCKS], dtype=np.int32)
    slots = [slot_of(table[0], p, bs) for p in range(L)]
    others = [b for b in range(nb) if b not in WORKED_EXAMPLE_BLOCKS]
    other_live = np.zeros((nb, bs), dtype=bool)
    other_live[others[:len(others) // 2]] = True     # other requests' rows
    return _build("worked_example", rng, q_kind="f32", kv_kind="f32",
                  src_kind="f32", hq=1, hkv=1, d=d, bs=bs, nb=nb,
                  block_tables=table, seq_lens=[L], cached_lens=[0],
                  slot_mapping=slots, copy_pairs=np.zeros((0, 2)),
                  live_extra=other_live,
                  note="page-2 figure: bs 4, 22 tokens on blocks 7,2,11,5,9,0")


def llama8b_decode(num_seqs=32, median=512, cap=4096, num_blocks=16384,
                   replicas=1, seed_family=1):
    """Llama-3-8B-shaped decode layer: 32 sequences, 32/8 heads, D 128,
    bs 16, bf16; lognormal lengths (median 512, cap 4096); block ids from a
    random permutation of a 16384-block pool; 1 new token per sequence.
    ``replicas`` > 1 adds disjoint id sets over the same pool."""
    rng = np.random.default_rng([SEED_BASE, seed_family])
    bs = 16
    lens = lognormal_lengths(rng, num_seqs, median, cap)
    perm = rng.permutation(num_blocks).astype(np.int32)
    filler = int(perm[-1])                       # never handed out: poison
    max_blocks = blocks_for(cap, bs)
    need = sum(blocks_for(L, bs) for L in lens)
    replicas = max(1, min(replicas, (num_blocks - 1) // max(need, 1)))
    sets = []
    for r in range(replicas):
        tables, slots, _ = _decode_layout(lens, bs, perm[r * need:(r + 1) * need],
                                          max_blocks, filler)
        sets.append({"block_tables": tables, "slot_mapping": slots,
                     "copy_pairs": np.zeros((0, 2), dtype=np.int32)})
    cached = [int(L) - 1 for L in lens]
    return _build("llama8b_decode", rng, q_kind="bf16", kv_kind="bf16",
                  src_kind="bf16", hq=32, hkv=8, d=128, bs=bs, nb=num_blocks,
                  block_tables=sets[0]["block_tables"], seq_lens=lens,
                  cached_lens=cached, slot_mapping=sets[0]["slot_mapping"],
                  copy_pairs=sets[0]["copy_pairs"], replicas=sets[1:],
                  note=f"{len(sets)} disjoint replica(s)")


def llama70b_decode(num_seqs=256, median=1024, cap=8192, occupancy=0.9,
                    seed_family=2):
    """70B-shaped decode layer at high concurrency: 256 sequences, 64/8
    heads, D 128, bs 16, fp16; lognormal lengths (median 1024, cap 8192);
    scattered blocks in a pool sized to 90 % occupancy; 256 new tokens."""
    rng = np.random.default_rng([SEED_BASE, seed_family])
    bs = 16
    lens = lognormal_lengths(rng, num_seqs, median, cap)
    used = sum(blocks_for(L, bs) for L in lens)
    nb = int(math.ceil(used / occupancy))
    if nb == used:
        nb += 1
    perm = rng.permutation(nb).astype(np.int32)
    filler = int(perm[-1])
    tables, slots, _ = _decode_layout(lens, bs, perm, blocks_for(cap, bs),
                                      filler)
    cached = [int(L) - 1 for L in lens]
    return _build("llama70b_decode", rng, q_kind="f16", kv_kind="f16",
                  src_kind="f16", hq=64, hkv=8, d=128, bs=bs, nb=nb,
                  block_tables=tables, seq_lens=lens, cached_lens=cached,
                  slot_mapping=slots, copy_pairs=np.zeros((0, 2)),
                  note=f"pool {nb} blocks, {used} used")


def prefix_sharing(block_size=32, phase="fork", groups=8, samples=8,
                   prompt_len=2048, max_tail=512, seed_family=3):
    """Parallel sampling with a shared prompt: ``groups`` prompts of
    ``prompt_len`` tokens, ``samples`` samples each (refcount = samples on
    the prompt's blocks), 32/8 heads, D 128, bf16.

    phase "fork": every sample appends its first token (position
    prompt_len).  If the prompt's last block is partial it is shared, so
    each sample but the last copies it into a fresh block before writing;
    the last sample finds a reference count of 1 and writes in place
    ("Sharing and copy-on-write": at most one copy per sequence, only of a
    partial block).  With a block-aligned prompt no copy is needed.

    phase "divergent": the state after the fork plus ``t ~ U{0..max_tail}``
    private tail tokens per sample; each appends one token at position
    prompt_len + t.  The prompt's full blocks stay shared.
    """
    assert phase in ("fork", "divergent")
    rng = np.random.default_rng([SEED_BASE, seed_family])
    bs = block_size
    S = groups * samples
    tails = rng.integers(0, max_tail + 1, size=S) if phase == "divergent" \
        else np.zeros(S, dtype=np.int64)
    full_prompt, rem = divmod(prompt_len, bs)
    prompt_blocks = full_prompt + (1 if rem else 0)
    lens = prompt_len + tails + 1
    # blocks needed: shared prompt blocks per group + private blocks per sample
    priv_counts = [blocks_for(L, bs) - full_prompt for L in lens]
    need = groups * prompt_blocks + sum(priv_counts)
    nb = 2 * need
    perm = rng.permutation(nb).astype(np.int32)
    free = list(perm)
    filler = int(free.pop())            # reserved poison block
    max_blocks = blocks_for(prompt_len + max_tail + 1, bs)
    tables = np.full((S, max_blocks), filler, dtype=np.int32)
    pairs = []
    extra_live = np.zeros((nb, bs), dtype=bool)
    prompt_tables = []
    for g in range(groups):
        ids = [free.pop(0) for _ in range(prompt_blocks)]
        prompt_tables.append(ids)
        for j in range(full_prompt):
            extra_live[ids[j]] = True
        if rem:
            extra_live[ids[full_prompt], :rem] = True
    slots = []
    cached_for_live = []
    for g in range(groups):
        shared = prompt_tables[g]
        refcount_partial = samples
        for k in range(samples):
            s = g * samples + k
            L = int(lens[s])
            row = tables[s]
            row[:full_prompt] = shared[:full_prompt]
            n_total = blocks_for(L, bs)
            if rem:
                if phase == "fork":
                    if refcount_partial > 1:
                        dst = free.pop(0)
                        pairs.append((shared[full_prompt], dst))
                        refcount_partial -= 1
                        row[full_prompt] = dst
                    else:
                        row[full_prompt] = shared[full_prompt]
                elif k < samples - 1:
                    # samples that copied the prompt's partial block at
                    # their fork step own a private copy of it
                    own = free.pop(0)
                    row[full_prompt] = own
                    extra_live[own, :rem] = True
                else:
                    # the last sample kept the original (refcount 1)
                    row[full_prompt] = shared[full_prompt]
                start = full_prompt + 1
            else:
                start = full_prompt
            for j in range(start, n_total):
                row[j] = free.pop(0)
            # private tail tokens already cached (positions prompt_len ..
            # L-2) are live
            for p in range(prompt_len, L - 1):
                extra_live[row[p // bs], p % bs] = True
            slots.append(slot_of(row, L - 1, bs))
            cached_for_live.append(0)
    name = f"prefix_sharing_{phase}_bs{bs}"
    note = f"{groups}x{samples} samples, {len(pairs)} copy pairs"
    return _build(name, rng, q_kind="bf16", kv_kind="bf16", src_kind="bf16",
                  hq=32, hkv=8, d=128, bs=bs, nb=nb, block_tables=tables,
                  seq_lens=lens, cached_lens=cached_for_live,
                  slot_mapping=slots, copy_pairs=pairs,
                  live_extra=extra_live,
                  note=note), prompt_tables


def long_context_fp8(num_seqs=8, seq_len=131072, block_size=64,
                     seed_family=4, per_token_scales=False):
    """Long-context split-K decode: 8 sequences of 131072 tokens, 32/8
    heads, D 128, bs 64; K/V cached as fp8 E4M3 with per-tensor scales
    (max|live value| / 448; with per_token_scales one per (slot, kv head)
    instead), Q and the new rows bf16.  Blocks are a random permutation of
    the used blocks plus one poisoned spare for unused table columns.  (How
    each sequence is split for the log-sum-exp merge is the kernel's choice,
    not part of the inputs.)"""
    rng = np.random.default_rng([SEED_BASE, seed_family])
    bs = block_size
    lens = np.full(num_seqs, seq_len, dtype=np.int64)
    used = num_seqs * blocks_for(seq_len, bs)
    nb = used + 1
    perm = rng.permutation(used).astype(np.int32)
    filler = used                                   # the spare block
    tables, slots, _ = _decode_layout(lens, bs, perm, blocks_for(seq_len, bs),
                                      filler)
    cached = [int(L) - 1 for L in lens]
    return _build("long_context_fp8", rng, q_kind="bf16", kv_kind="fp8_e4m3",
                  src_kind="bf16", hq=32, hkv=8, d=128, bs=bs, nb=nb,
                  block_tables=tables, seq_lens=lens, cached_lens=cached,
                  slot_mapping=slots, copy_pairs=np.zeros((0, 2)),
                  note=f"{used} used blocks + 1 spare",
                  per_token_scales=per_token_scales)


def custom_decode(*, seed, num_seqs, lens, hq, hkv, d, bs, q_kind, kv_kind,
                  src_kind=None, spare_blocks=3, num_new_per_seq=1,
                  per_head_scales=False, per_token_scales=False):
    """Small free-form decode step (fuzz/edge cases): lengths given, blocks
    from a random permutation with a few spare poisoned blocks; an fp8
    cache's scales per tensor, per kv head (per_head_scales) or per (slot,
    kv head) (per_token_scales)."""
    rng = np.random.default_rng([SEED_BASE, 100, seed])
    src_kind = src_kind or (q_kind if kv_kind in FP8_KINDS else kv_kind)
    lens = np.asarray(lens, dtype=np.int64)
    need = sum(blocks_for(max(int(L), 1), bs) for L in lens)  # (an empty
    # sequence still gets a table row laid out over one block)
    nb = need + spare_blocks
    perm = rng.permutation(nb).astype(np.int32)
    filler = int(perm[-1])
    max_blocks = max(1, max(blocks_for(L, bs) for L in lens)) if len(lens) \
        else 1
    tables, _, _ = _decode_layout(np.maximum(lens, 1), bs, perm, max_blocks,
                                  filler)
    for i, L in enumerate(lens):
        if L == 0:
            tables[i, :] = filler
    slots = []
    for i, L in enumerate(lens):
        L = int(L)
        for p in range(max(0, L - num_new_per_seq), L):
            slots.append(slot_of(tables[i], p, bs))
    cached = [max(0, int(L) - num_new_per_seq) for L in lens]
    return _build(f"custom_{seed}", rng, q_kind=q_kind, kv_kind=kv_kind,
                  src_kind=src_kind, hq=hq, hkv=hkv, d=d, bs=bs, nb=nb,
                  block_tables=tables, seq_lens=lens, cached_lens=cached,
                  slot_mapping=slots, copy_pairs=np.zeros((0, 2)),
                  per_head_scales=per_head_scales,
                  per_token_scales=per_token_scales)


# ----------------------------------------------------------------------------
# several new query tokens per sequence (chunked prefill, draft verification)
# ----------------------------------------------------------------------------

@dataclass
class MultiQuery:
    """A step with qlens[s] new tokens per sequence: ``w`` holds the pools
    before the step (the new tokens' slots poisoned), the tables, the lengths
    after it, and the new rows (``w.key``/``w.value``/``w.slot_mapping``,
    sequence after sequence); ``query`` [T, Hq, D] has one row per new token
    in the same order, and ``query_start`` [S + 1] the exclusive prefix of
    qlens."""
    w: Workload
    query: np.ndarray
    query_start: np.ndarray

    @property
    def max_query_len(self):
        q = np.diff(self.query_start)
        return int(q.max()) if len(q) else 0


def _multi(name, rng, *, lens, qlens, hq, hkv, d, bs, q_kind, kv_kind,
           src_kind, nb, perm, replicas=1, per_head_scales=False,
           per_token_scales=False):
    lens = np.asarray(lens, dtype=np.int64)
    qlens = np.asarray(qlens, dtype=np.int64)
    assert (qlens <= lens).all() and (qlens >= 0).all()
    filler = int(perm[-1])
    max_blocks = max(1, max(blocks_for(L, bs) for L in lens))
    need = sum(blocks_for(max(int(L), 1), bs) for L in lens)
    sets = []
    for r in range(replicas):
        tables, _, _ = _decode_layout(np.maximum(lens, 1), bs,
                                      perm[r * need:(r + 1) * need],
                                      max_blocks, filler)
        for i, L in enumerate(lens):
            if L == 0:
                tables[i, :] = filler
        slots = [slot_of(tables[i], p, bs) for i, L in enumerate(lens)
                 for p in range(int(L - qlens[i]), int(L))]
        sets.append({"block_tables": tables, "slot_mapping": slots,
                     "copy_pairs": np.zeros((0, 2), dtype=np.int32)})
    cached = [int(L - q) for L, q in zip(lens, qlens)]
    w = _build(name, rng, q_kind=q_kind, kv_kind=kv_kind, src_kind=src_kind,
               hq=hq, hkv=hkv, d=d, bs=bs, nb=nb,
               block_tables=sets[0]["block_tables"], seq_lens=lens,
               cached_lens=cached, slot_mapping=sets[0]["slot_mapping"],
               copy_pairs=np.zeros((0, 2)), replicas=sets[1:],
               per_head_scales=per_head_scales,
               per_token_scales=per_token_scales)
    T = int(qlens.sum())
    query = _cast_from_f32(_normal(rng, (T, hq, d)), q_kind)
    query_start = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return MultiQuery(w=w, query=query, query_start=query_start)


def custom_multi(*, seed, lens, qlens, hq, hkv, d, bs, q_kind, kv_kind,
                 src_kind=None, spare_blocks=3, per_head_scales=False,
                 per_token_scales=False):
    """Small free-form multi-query step: lengths (after the step) and new
    tokens per sequence given; blocks from a random permutation."""
    rng = np.random.default_rng([SEED_BASE, 200, seed])
    src_kind = src_kind or (q_kind if kv_kind in FP8_KINDS else kv_kind)
    need = sum(blocks_for(max(int(L), 1), bs) for L in lens)
    nb = need + spare_blocks
    perm = rng.permutation(nb).astype(np.int32)
    return _multi(f"custom_multi_{seed}", rng, lens=lens, qlens=qlens, hq=hq,
                  hkv=hkv, d=d, bs=bs, q_kind=q_kind, kv_kind=kv_kind,
                  src_kind=src_kind, nb=nb, perm=perm,
                  per_head_scales=per_head_scales,
                  per_token_scales=per_token_scales)


def spec_verify_llama8b(num_seqs=32, draft=4, median=512, cap=4096,
                        num_blocks=16384, replicas=1, seed_family=6):
    """Speculative-decoding verification on the Llama-3-8B decode shape:
    32 sequences, 32/8 heads, D 128, bs 16, bf16, cached lengths lognormal
    (median 512, cap 4096) as in the decode batch, plus ``draft`` new tokens
    per sequence (the drafted tokens the target model scores in one pass,
    each seeing the cache and the drafts before it).  Block ids from a random
    permutation of a 16384-block pool; ``replicas`` > 1 adds disjoint id
    sets over the same pool."""
    rng = np.random.default_rng([SEED_BASE, seed_family])
    lens = lognormal_lengths(rng, num_seqs, median, cap - draft) + draft
    qlens = np.full(num_seqs, draft, dtype=np.int64)
    perm = rng.permutation(num_blocks).astype(np.int32)
    need = sum(blocks_for(int(L), 16) for L in lens)
    replicas = max(1, min(replicas, (num_blocks - 1) // max(need, 1)))
    return _multi("spec_verify_llama8b", rng, lens=lens, qlens=qlens, hq=32,
                  hkv=8, d=128, bs=16, q_kind="bf16", kv_kind="bf16",
                  src_kind="bf16", nb=num_blocks, perm=perm,
                  replicas=replicas)


def chunked_prefill_llama8b(num_seqs=8, prefix=4096, chunk=512,
                            num_blocks=16384, replicas=1, seed_family=7):
    """Chunked prefill on the Llama-3-8B layer shape: 8 sequences whose
    first ``prefix`` prompt tokens are already cached take the next
    ``chunk`` prompt tokens in one pass (causal among them); 32/8 heads,
    D 128, bs 16, bf16, blocks from a random permutation of a 16384-block
    pool."""
    rng = np.random.default_rng([SEED_BASE, seed_family])
    lens = np.full(num_seqs, prefix + chunk, dtype=np.int64)
    qlens = np.full(num_seqs, chunk, dtype=np.int64)
    perm = rng.permutation(num_blocks).astype(np.int32)
    need = num_seqs * blocks_for(prefix + chunk, 16)
    replicas = max(1, min(replicas, (num_blocks - 1) // need))
    return _multi("chunked_prefill_llama8b", rng, lens=lens, qlens=qlens,
                  hq=32, hkv=8, d=128, bs=16, q_kind="bf16", kv_kind="bf16",
                  src_kind="bf16", nb=num_blocks, perm=perm,
                  replicas=replicas)


MULTI_WORKLOADS = {"spec_verify_llama8b": spec_verify_llama8b,
                   "chunked_prefill_llama8b": chunked_prefill_llama8b}


# ----------------------------------------------------------------------------
# relabelling (for the block-permutation invariance check)
# ----------------------------------------------------------------------------

def permute_physical(w, perm):
    """Move physical block b to perm[b] everywhere: pools, tables, slots and
    copy pairs.  Logical content is unchanged."""
    perm = np.asarray(perm, dtype=np.int64)
    inv_pool_k = np.empty_like(w.k_pool)
    inv_pool_v = np.empty_like(w.v_pool)
    inv_pool_k[perm] = w.k_pool
    inv_pool_v[perm] = w.v_pool
    bs = w.block_size
    slots = w.slot_mapping.astype(np.int64)
    new_slots = np.where(slots >= 0, perm[np.maximum(slots, 0) // bs] * bs +
                         np.maximum(slots, 0) % bs, slots)
    return replace(w, k_pool=inv_pool_k, v_pool=inv_pool_v,
                   block_tables=perm[w.block_tables].astype(np.int32),
                   slot_mapping=new_slots.astype(np.int32),
                   copy_pairs=perm[w.copy_pairs.astype(np.int64)].astype(
                       np.int32).reshape(-1, 2),
                   replicas=[])


def workload_by_name(name, **kw):
    """Named workload families, sized as in the headline configurations."""
    if name == "worked_example":
        return worked_example(**kw)
    if name == "llama8b_decode":
        return llama8b_decode(**kw)
    if name == "llama70b_decode":
        return llama70b_decode(**kw)
    if name.startswith("prefix_sharing_"):
        _, _, phase, bs = name.split("_")
        return prefix_sharing(block_size=int(bs[2:]), phase=phase, **kw)[0]
    if name == "long_context_fp8":
        return long_context_fp8(**kw)
    raise KeyError(name)


# decode workloads workload_by_name knows (one new token per sequence)
DECODE_WORKLOADS = ("worked_example", "llama8b_decode", "llama70b_decode",
                    "prefix_sharing_fork_bs32", "prefix_sharing_fork_bs544",
                    "prefix_sharing_divergent_bs32",
                    "prefix_sharing_divergent_bs544", "long_context_fp8")
