"""Paged attention for several new query tokens per sequence — test
infrastructure only.

The method's read path ("PagedAttention", shubhamtatvamasi.com, section "How
attention reads paged memory") walks a sequence's block table and attends
over its gathered keys and values.  With more than one new token per
sequence -- a chunk of a prompt processed against an already cached prefix,
or the draft tokens a speculative decoder verifies -- each new token attends
to every token up to and including itself.  Reading (the pages cover one
query per sequence only): sequence s holds L_s tokens, its last q_s tokens
are the new ones (their keys and values are already in the cache), and new
token j (0-based) sits at position L_s - q_s + j and sees tokens
0 .. L_s - q_s + j (causal within the new tokens, everything before them).

Queries are packed sequence after sequence: rows query_start[s] ..
query_start[s+1]-1 of ``query`` belong to sequence s.  Everything else
(pool layout, head mapping, scales, float64 two-pass softmax) is as in
:mod:`oracle.attention`.
"""

import numpy as np

from .attention import attention_one_head, stored_rows
from .storage import to_float64


def paged_attention_multi(query, q_kind, k_pool, v_pool, kv_kind,
                          block_tables, seq_lens, query_start, block_size,
                          scale, k_scale=1.0, v_scale=1.0):
    """float64 [T, Hq, D] for query [T, Hq, D], T = query_start[-1]."""
    T, Hq, D = query.shape
    Hkv = k_pool.shape[2]
    G = Hq // Hkv
    q64 = to_float64(query, q_kind)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        nq = q1 - q0
        assert 0 <= nq <= L
        if nq == 0:
            continue
        for h in range(Hkv):
            k = stored_rows(k_pool, kv_kind, block_tables[s], L,
                            block_size, h, k_scale)
            v = stored_rows(v_pool, kv_kind, block_tables[s], L,
                            block_size, h, v_scale)
            for j in range(nq):
                p = L - nq + j
                out[q0 + j, h * G:(h + 1) * G] = attention_one_head(
                    q64[q0 + j, h * G:(h + 1) * G], k[:p + 1], v[:p + 1],
                    scale)
    return out
