"""Paged decode attention, written as its plain definition — test infrastructure.

Source: "PagedAttention" (shubhamtatvamasi.com), section "How attention reads
paged memory" and the figure beside it.  A decode query of one sequence sees
that sequence's tokens 0..L-1; logical block i of the sequence lives in
physical block ``block_table[i]`` of a per-layer pool shaped
``[num_blocks, block_size, kv_heads, head_dim]``, and token j sits at
offset ``j % block_size`` of logical block ``j // block_size``.  Paging only
changes where the rows live, so paged attention equals ordinary softmax
attention over the sequence's keys and values gathered back into logical
order — that is what this module computes, in float64, with two passes
(maximum first, then exponentials and sums) rather than the kernel's online
update.

Readings of points the pages leave open (each also listed in the design
notes):

* the softmax scale is an explicit argument (the workloads use 1/sqrt(D));
* with ``Hq`` query heads over ``Hkv`` cache heads, query head ``h`` reads
  cache head ``h // (Hq // Hkv)`` (contiguous groups);
* ``seq_lens`` counts the token written in the same step, and no other
  mask applies; a sequence of length 0 yields zeros;
* fp8 caches (E4M3 or E5M2) hold codes of ``x / scale``; the stored value
  is ``decode(code) * scale`` (the scale is applied exactly in float64);
  the scale is per tensor, one per kv head, or one per (token slot, kv
  head) -- a float32 array shaped like the pool without its head_dim axis,
  ``[num_blocks, block_size, kv_heads]``, written beside each row;
* the output is returned in float64 (the GPU path writes float32).
"""

import numpy as np

from .storage import FP8_KINDS, head_scales, to_float64


def gather_sequence(pool, table_row, seq_len, block_size, head):
    """Rows 0..seq_len-1 of one sequence for cache head ``head``: [L, D].

    Walks the block table: logical block i -> physical block table_row[i],
    concatenated in logical order, cut to the first ``seq_len`` tokens.
    """
    n_blocks = -(-int(seq_len) // int(block_size))
    phys = np.asarray(table_row[:n_blocks], dtype=np.int64)
    blocks = pool[phys, :, head, :]                 # [n, bs, D]
    rows = blocks.reshape(n_blocks * block_size, pool.shape[3])
    return rows[:seq_len]


def is_token_scales(scale):
    """True for per-token scales: a [num_blocks, block_size, kv_heads]
    array (one float32 per slot and kv head)."""
    return np.ndim(scale) == 3


def stored_rows(pool, kind, table_row, seq_len, block_size, head, scale):
    """The values one sequence's rows of cache head ``head`` stand for, in
    float64 [L, D]: the gathered storage widened exactly, times the fp8
    scale that applies to each row (per tensor, per kv head, or the row's
    own per-token scale gathered through the same table walk)."""
    rows = to_float64(gather_sequence(pool, table_row, seq_len, block_size,
                                      head), kind)
    if kind not in FP8_KINDS:
        return rows
    if is_token_scales(scale):
        sc = np.asarray(scale, dtype=np.float32)[..., None]  # [nb, bs, Hkv, 1]
        per_row = gather_sequence(sc, table_row, seq_len, block_size, head)
        return rows * per_row.astype(np.float64)
    return rows * head_scales(scale, pool.shape[2])[head]


def attention_one_head(q, k, v, scale):
    """softmax(scale * q k^T) v for a block of query rows, in float64.

    q: [G, D], k: [L, D], v: [L, D]  ->  [G, D].
    Pass 1 takes the row maximum of the scores; pass 2 forms
    exp(score - max), its sum, and the weighted sum of value rows.
    """
    scores = scale * (q @ k.T)                      # [G, L]
    m = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - m)
    denom = p.sum(axis=1, keepdims=True)
    return (p @ v) / denom


def paged_attention(query, q_kind, k_pool, v_pool, kv_kind, block_tables,
                    seq_lens, block_size, scale, k_scale=1.0, v_scale=1.0):
    """Decode attention for every sequence and query head -> float64 [S, Hq, D].

    query: [S, Hq, D] storage array of kind ``q_kind``.
    k_pool, v_pool: [num_blocks, block_size, Hkv, D] of kind ``kv_kind``.
    block_tables: int32 [S, max_blocks]; only the first ceil(L/bs) columns
    of a row are read.  seq_lens: int32 [S].
    k_scale, v_scale: per-tensor scales, one per kv head, or per-token
    scale arrays [num_blocks, block_size, Hkv], used only for fp8 caches.
    """
    S, Hq, D = query.shape
    Hkv = k_pool.shape[2]
    assert Hq % Hkv == 0
    assert k_pool.shape[1] == block_size
    G = Hq // Hkv
    q64 = to_float64(query, q_kind)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L == 0:
            continue
        for h in range(Hkv):
            k = stored_rows(k_pool, kv_kind, block_tables[s], L, block_size,
                            h, k_scale)
            v = stored_rows(v_pool, kv_kind, block_tables[s], L, block_size,
                            h, v_scale)
            out[s, h * G:(h + 1) * G] = attention_one_head(
                q64[s, h * G:(h + 1) * G], k, v, scale)
    return out


def paged_attention_rows(query, q_kind, k_pool, v_pool, kv_kind, block_tables,
                         seq_lens, block_size, scale, rows, k_scale=1.0,
                         v_scale=1.0):
    """:func:`paged_attention` for the (seq, q_head) pairs in ``rows`` only;
    returns float64 [len(rows), D], row i being ``paged_attention(...)[s,
    hq]`` of ``rows[i] = (s, hq)`` bit for bit.  The pairs are grouped by
    (sequence, kv head): each group's rows are gathered once, and all G
    query heads of that kv head go through the same float64 computation as
    in :func:`paged_attention`, of which the asked-for heads are kept.  Used
    to check full-size workloads, whose whole output would not fit the
    oracle's time, sequence by sequence or on sampled pairs."""
    S, Hq, D = query.shape
    Hkv = k_pool.shape[2]
    assert Hq % Hkv == 0
    assert k_pool.shape[1] == block_size
    G = Hq // Hkv
    out = np.zeros((len(rows), D), dtype=np.float64)
    groups = {}
    for i, (s, hq) in enumerate(rows):
        groups.setdefault((int(s), int(hq) // G), []).append((i, int(hq)))
    for (s, h), members in groups.items():
        L = int(seq_lens[s])
        if L == 0:
            continue
        k = stored_rows(k_pool, kv_kind, block_tables[s], L, block_size, h,
                        k_scale)
        v = stored_rows(v_pool, kv_kind, block_tables[s], L, block_size, h,
                        v_scale)
        q = to_float64(query[s, h * G:(h + 1) * G], q_kind)
        o = attention_one_head(q, k, v, scale)
        for i, hq in members:
            out[i] = o[hq - h * G]
    return out
