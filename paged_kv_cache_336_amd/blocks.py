"""Python binding of the host block manager (include/pagedkv_blocks.h).

Argument marshalling only: every decision is made by the C++ manager in
libpagedkv.so.  A failed call raises ``BlockError`` carrying the library's
status code; ``NoFreeBlocks`` is its subclass for ``PKV_ERR_NO_BLOCKS``.
"""

import ctypes

import numpy as np

from . import ops

PKV_ERR_NO_BLOCKS = 9

EXPORTED = ("pkv_bm_create", "pkv_bm_create_prefix_cached",
            "pkv_bm_add_sequence_tokens", "pkv_bm_prefix_stats",
            "pkv_bm_destroy", "pkv_bm_add_sequence",
            "pkv_bm_fork", "pkv_bm_append", "pkv_bm_free", "pkv_bm_tables",
            "pkv_bm_blocks_unshared",
            "pkv_bm_get_stats", "pkv_bm_refcount", "pkv_bm_seq_len",
            "pkv_ca_create", "pkv_ca_destroy", "pkv_ca_reserve",
            "pkv_ca_release", "pkv_ca_get_stats")


class BlockError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {ops.pkv_status_string(status)} "
                         f"(status {status})")
        self.status = status


class NoFreeBlocks(BlockError):
    pass


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "free_blocks", "used_blocks", "shared_blocks", "live_sequences",
        "logical_tokens", "stored_tokens", "wasted_slots")]


_typed = False


def _lib():
    global _typed
    lib = ops.load_library()
    if not _typed:
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        ci = ctypes.c_int
        lib.pkv_bm_create.restype = vp
        lib.pkv_bm_create.argtypes = [i32, i32, i32, i32]
        lib.pkv_bm_create_prefix_cached.restype = vp
        lib.pkv_bm_create_prefix_cached.argtypes = [i32, i32, i32, i32]
        lib.pkv_bm_add_sequence_tokens.restype = ci
        lib.pkv_bm_add_sequence_tokens.argtypes = [vp, i32, vp, i32, vp, vp]
        lib.pkv_bm_prefix_stats.restype = ci
        lib.pkv_bm_prefix_stats.argtypes = [vp, ctypes.POINTER(i64),
                                            ctypes.POINTER(i64),
                                            ctypes.POINTER(i64)]
        lib.pkv_bm_destroy.restype = None
        lib.pkv_bm_destroy.argtypes = [vp]
        lib.pkv_bm_add_sequence.restype = ci
        lib.pkv_bm_add_sequence.argtypes = [vp, i32, i32, vp]
        lib.pkv_bm_fork.restype = ci
        lib.pkv_bm_fork.argtypes = [vp, i32, i32]
        lib.pkv_bm_append.restype = ci
        lib.pkv_bm_append.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        lib.pkv_bm_free.restype = ci
        lib.pkv_bm_free.argtypes = [vp, i32]
        lib.pkv_bm_tables.restype = ci
        lib.pkv_bm_tables.argtypes = [vp, vp, i32, vp, i32, i32, vp]
        lib.pkv_bm_blocks_unshared.restype = ci
        lib.pkv_bm_blocks_unshared.argtypes = [vp, vp, i32,
                                               ctypes.POINTER(i32)]
        lib.pkv_bm_get_stats.restype = ci
        lib.pkv_bm_get_stats.argtypes = [vp, ctypes.POINTER(_Stats)]
        lib.pkv_bm_refcount.restype = i32
        lib.pkv_bm_refcount.argtypes = [vp, i32]
        lib.pkv_bm_seq_len.restype = i32
        lib.pkv_bm_seq_len.argtypes = [vp, i32]
        lib.pkv_ca_create.restype = vp
        lib.pkv_ca_create.argtypes = [i64, i32]
        lib.pkv_ca_destroy.restype = None
        lib.pkv_ca_destroy.argtypes = [vp]
        lib.pkv_ca_reserve.restype = ci
        lib.pkv_ca_reserve.argtypes = [vp, i32, i64, ctypes.POINTER(i64)]
        lib.pkv_ca_release.restype = ci
        lib.pkv_ca_release.argtypes = [vp, i32]
        lib.pkv_ca_get_stats.restype = ci
        lib.pkv_ca_get_stats.argtypes = [vp, ctypes.POINTER(i64),
                                         ctypes.POINTER(i64),
                                         ctypes.POINTER(i64)]
        _typed = True
    return lib


def _check(status, what):
    if status == 0:
        return
    cls = NoFreeBlocks if status == PKV_ERR_NO_BLOCKS else BlockError
    raise cls(status, what)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


class BlockManager:
    """Physical-block bookkeeping for one paged pool (see pagedkv_blocks.h)."""

    def __init__(self, num_blocks, block_size, max_seqs, max_blocks_per_seq,
                 prefix_cache=False):
        self.lib = _lib()
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        create = (self.lib.pkv_bm_create_prefix_cached if prefix_cache
                  else self.lib.pkv_bm_create)
        self.h = create(num_blocks, block_size, max_seqs, max_blocks_per_seq)
        if not self.h:
            raise ValueError("pkv_bm_create rejected its arguments")

    def close(self):
        if self.h:
            self.lib.pkv_bm_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def add_sequence(self, seq, num_tokens):
        """Slots (int32 [num_tokens]) of the prompt's tokens."""
        slots = np.empty(max(num_tokens, 1), dtype=np.int32)
        _check(self.lib.pkv_bm_add_sequence(self.h, seq, num_tokens,
                                            _ptr(slots)), "add_sequence")
        return slots[:num_tokens]

    def add_sequence_tokens(self, seq, tokens):
        """A prompt given by its token ids: (slots int32 [n], the number of
        leading tokens whose blocks came from the prefix cache)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        n = len(toks)
        slots = np.empty(max(n, 1), dtype=np.int32)
        cached = ctypes.c_int32(0)
        _check(self.lib.pkv_bm_add_sequence_tokens(
            self.h, seq, _ptr(toks) if n else None, n, _ptr(slots),
            ctypes.byref(cached)), "add_sequence_tokens")
        return slots[:n], int(cached.value)

    def prefix_stats(self):
        r, e, h = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(self.lib.pkv_bm_prefix_stats(self.h, ctypes.byref(r),
                                            ctypes.byref(e), ctypes.byref(h)),
               "prefix_stats")
        return {"registered": r.value, "evictable": e.value,
                "hit_blocks": h.value}

    def fork(self, parent, child):
        _check(self.lib.pkv_bm_fork(self.h, parent, child), "fork")

    def append(self, seqs, with_counts=False):
        """One token for each sequence: (slot_mapping int32 [n], copy pairs
        int32 [p, 2]) and, with_counts, the tokens each copy carries
        (int32 [p]; rows {src, dst, tokens} for copy_block_prefixes)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = len(seqs)
        slots = np.empty(max(n, 1), dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        counts = np.empty(max(n, 1), dtype=np.int32)
        npairs = ctypes.c_int32(0)
        _check(self.lib.pkv_bm_append(self.h, _ptr(seqs), n, _ptr(slots),
                                      _ptr(pairs), ctypes.byref(npairs),
                                      _ptr(counts)),
               "append")
        p = npairs.value
        if with_counts:
            return slots[:n], pairs[:p].copy(), counts[:p].copy()
        return slots[:n], pairs[:p].copy()

    def free(self, seq):
        _check(self.lib.pkv_bm_free(self.h, seq), "free")

    def tables(self, seqs, fill=0, row_stride=None):
        """(block_tables int32 [n, row_stride], seq_lens int32 [n])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        stride = row_stride or self.max_blocks_per_seq
        tab = np.empty((len(seqs), stride), dtype=np.int32)
        lens = np.empty(len(seqs), dtype=np.int32)
        _check(self.lib.pkv_bm_tables(self.h, _ptr(seqs), len(seqs),
                                      _ptr(tab), stride, fill, _ptr(lens)),
               "tables")
        return tab, lens

    def blocks_unshared(self, seqs):
        """True when no physical block appears in two of these sequences'
        tables: an attention call over them may pass PKV_KV_STREAM."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        out = ctypes.c_int32(-1)
        _check(self.lib.pkv_bm_blocks_unshared(self.h, _ptr(seqs), len(seqs),
                                               ctypes.byref(out)),
               "blocks_unshared")
        return bool(out.value)

    def stats(self):
        st = _Stats()
        _check(self.lib.pkv_bm_get_stats(self.h, ctypes.byref(st)), "stats")
        return {n: int(getattr(st, n)) for n, _ in _Stats._fields_}

    def refcount(self, block):
        return int(self.lib.pkv_bm_refcount(self.h, block))

    def seq_len(self, seq):
        return int(self.lib.pkv_bm_seq_len(self.h, seq))


class ContiguousAllocator:
    """Max-length reservations, first fit (the baseline paging replaces)."""

    def __init__(self, num_slots, max_requests):
        self.lib = _lib()
        self.h = self.lib.pkv_ca_create(num_slots, max_requests)
        if not self.h:
            raise ValueError("pkv_ca_create rejected its arguments")

    def close(self):
        if self.h:
            self.lib.pkv_ca_destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def reserve(self, req, num_slots):
        """Start slot, or None when no single gap fits."""
        start = ctypes.c_int64(-1)
        st = self.lib.pkv_ca_reserve(self.h, req, num_slots,
                                     ctypes.byref(start))
        if st == PKV_ERR_NO_BLOCKS:
            return None
        _check(st, "reserve")
        return int(start.value)

    def release(self, req):
        _check(self.lib.pkv_ca_release(self.h, req), "release")

    def stats(self):
        f, g, r = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(self.lib.pkv_ca_get_stats(self.h, ctypes.byref(f),
                                         ctypes.byref(g), ctypes.byref(r)),
               "stats")
        return {"free_slots": f.value, "largest_gap": g.value,
                "reserved_slots": r.value}
