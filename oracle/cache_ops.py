"""Slot-mapped cache write and copy-on-write block copy — test infrastructure.

Both functions return new arrays and leave their inputs untouched.

cache_write — "How PagedAttention Works in vLLM ..." (instagit.com), section
"write_to_paged_cache: Direct In-Place Updates" and the code example: new
key/value rows ``[T, kv_heads, head_dim]`` go, in place, to the flat slots
given by an int32 slot mapping, where slot = physical_block * block_size +
offset (the slot numbering follows the block/offset addressing of
"PagedAttention" (shubhamtatvamasi.com), "How attention reads paged memory").
Readings: a negative slot means "skip this token" (padding); when the cache
dtype equals the source dtype the row is copied bit for bit; for an fp8
cache each element becomes ``enc(float32(x) / float32(scale))`` with an
IEEE float32 division and the round-to-nearest-even encoder of
:mod:`oracle.fp8_e4m3` (saturating) or :mod:`oracle.fp8_e5m2` (IEEE
overflow).  The scale is per tensor, or one per kv head (the pages' 0-d
scale tensors generalised; element ``[h, d]`` of a row uses scale ``h``).

cache_write_token_scales -- the same write with a scale per token row
(reading: the pages' scale is per tensor; here each written (token, kv
head) row picks its own, so that one large row does not coarsen the others).
The row's scale is its largest magnitude (NaN ignored; 0 when there is
none) over the format's largest finite value (448 for E4M3, 57344 for
E5M2), an IEEE float32 division, and 1 for a row without a nonzero
element; it is stored at the row's slot and head of a float32
``[num_blocks, block_size, kv_heads]`` array beside the pool, and the
row's codes are those of ``float32(x) / scale`` as above.

copy_blocks — "PagedAttention" (shubhamtatvamasi.com), "Sharing and
copy-on-write" and the FAQ entry on copy-on-write for parallel sampling:
before a sequence appends to a shared, partially filled block, the engine
copies that block into a fresh one.  The library's part is the copy: for
each (src, dst) pair, every slot of block ``dst`` in both pools takes the
contents of block ``src``.  Reading: the whole block is copied (the pairs
carry no token counts).
"""

import numpy as np

from .fp8_e4m3 import E4M3_MAX, e4m3_encode
from .fp8_e5m2 import E5M2_MAX, e5m2_encode
from .storage import head_scales, to_float64

_ENCODERS = {"fp8_e4m3": e4m3_encode, "fp8_e5m2": e5m2_encode}
_LARGEST = {"fp8_e4m3": E4M3_MAX, "fp8_e5m2": E5M2_MAX}


def _encode_row(row, src_kind, cache_kind, scale):
    """One token's row [Hkv, D] in the cache's storage."""
    if cache_kind == src_kind:
        return row.copy()
    if cache_kind in _ENCODERS:
        x32 = to_float64(row, src_kind).astype(np.float32)   # exact widening
        s32 = head_scales(scale, row.shape[0]).astype(np.float32)[:, None]
        y = x32 / s32                                         # IEEE fp32 div
        return _ENCODERS[cache_kind](y.astype(np.float64))
    raise ValueError(f"unsupported write {src_kind} -> {cache_kind}")


def cache_write(k_pool, v_pool, cache_kind, key, value, src_kind,
                slot_mapping, block_size, k_scale=1.0, v_scale=1.0):
    """Scatter new rows into copies of the pools; returns (k_pool, v_pool)."""
    kp = k_pool.copy()
    vp = v_pool.copy()
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        b, o = divmod(slot, int(block_size))
        kp[b, o] = _encode_row(key[t], src_kind, cache_kind, k_scale)
        vp[b, o] = _encode_row(value[t], src_kind, cache_kind, v_scale)
    return kp, vp


def token_row_scale(row32, cache_kind):
    """float32 scale of one written row (float32 [D])."""
    amax = np.float32(0.0)
    for x in np.abs(row32):
        amax = np.fmax(amax, x)            # NaN ignored, as fmax does
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax) / np.float32(_LARGEST[cache_kind])  # IEEE fp32


def cache_write_token_scales(k_pool, v_pool, k_scales, v_scales, cache_kind,
                             key, value, src_kind, slot_mapping, block_size):
    """Per-token-scaled fp8 write into copies of the pools and of their
    scale arrays; returns (k_pool, v_pool, k_scales, v_scales)."""
    assert cache_kind in _ENCODERS, cache_kind
    kp, vp = k_pool.copy(), v_pool.copy()
    ks = np.array(k_scales, dtype=np.float32, copy=True)
    vs = np.array(v_scales, dtype=np.float32, copy=True)
    enc = _ENCODERS[cache_kind]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        b, o = divmod(slot, int(block_size))
        for pool, scales, rows in ((kp, ks, key), (vp, vs, value)):
            x32 = to_float64(rows[t], src_kind).astype(np.float32)  # [Hkv, D]
            for h in range(x32.shape[0]):
                sc = token_row_scale(x32[h], cache_kind)
                scales[b, o, h] = sc
                pool[b, o, h] = enc((x32[h] / sc).astype(np.float64))
    return kp, vp, ks, vs


def copy_token_scales(k_scales, v_scales, records, prefix=False):
    """The per-token scale arrays follow their rows through a copy: with
    pairs (src, dst) whole blocks, with triples (src, dst, tokens) the
    first ``tokens`` slots (clamped to [0, block_size])."""
    ks = np.array(k_scales, copy=True)
    vs = np.array(v_scales, copy=True)
    bs = ks.shape[1]
    w = 3 if prefix else 2
    for rec in np.asarray(records, dtype=np.int64).reshape(-1, w):
        src, dst = int(rec[0]), int(rec[1])
        n = min(max(int(rec[2]), 0), bs) if prefix else bs
        ks[dst, :n] = ks[src, :n]
        vs[dst, :n] = vs[src, :n]
    return ks, vs


def copy_block_prefixes(k_pool, v_pool, triples):
    """Copies of the tokens a block holds (the FAQ entry on copy-on-write:
    the existing tokens go into the new block): for each (src, dst, tokens),
    slots 0 .. tokens-1 of dst take those of src in both pools; the rest of
    dst is left as it was.  Reading: tokens is clamped to [0, block_size]."""
    kp = k_pool.copy()
    vp = v_pool.copy()
    bs = k_pool.shape[1]
    for src, dst, n in np.asarray(triples, dtype=np.int64).reshape(-1, 3):
        n = min(max(int(n), 0), bs)
        kp[dst, :n] = kp[src, :n]
        vp[dst, :n] = vp[src, :n]
    return kp, vp


def copy_blocks(k_pool, v_pool, pairs):
    """Whole-block copies src -> dst in both pools; returns (k_pool, v_pool)."""
    kp = k_pool.copy()
    vp = v_pool.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        kp[dst] = kp[src]
        vp[dst] = vp[src]
    return kp, vp
