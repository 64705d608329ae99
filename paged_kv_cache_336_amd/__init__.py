"""MI355X-native paged KV-cache hot path: paged decode attention, the
slot-mapped cache write and the copy-on-write block copy.

The compute lives in ``libpagedkv.so`` (hand-written HIP for gfx950, C ABI
declared in ``include/pagedkv.h``).  :mod:`paged_kv_cache_336_amd.ops` is a
thin ctypes binding over it that takes torch tensors for device memory and
streams; it raises if the library is missing rather than computing anything
itself.  :mod:`paged_kv_cache_336_amd.workloads` builds seeded inputs.
"""

__all__ = ["ops", "workloads"]


def __getattr__(name):
    if name in ("ops", "workloads"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
