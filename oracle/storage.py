"""Exact widening of stored cache/query values to float64 — test infrastructure.

Storage kinds: ``"f32"`` (float32), ``"f16"`` (float16), ``"bf16"`` (uint16
holding the upper half of a float32 bit pattern), ``"fp8_e4m3"`` (uint8 OCP
E4M3 codes, decoded by :mod:`oracle.fp8_e4m3`), ``"fp8_e5m2"`` (uint8 OCP
E5M2 codes, decoded by :mod:`oracle.fp8_e5m2`).  Every conversion here is
exact: each stored value is representable in float64.
"""

import numpy as np

from .fp8_e4m3 import e4m3_decode
from .fp8_e5m2 import e5m2_decode

KINDS = ("f32", "f16", "bf16", "fp8_e4m3", "fp8_e5m2")
FP8_KINDS = ("fp8_e4m3", "fp8_e5m2")
_FP8_DECODERS = {"fp8_e4m3": e4m3_decode, "fp8_e5m2": e5m2_decode}
_FP8_TABLES = {}


def fp8_table(kind):
    """float64 [256]: the decoder's value of every code, in code order.
    Large arrays are widened by looking their codes up here, which gives
    the decoder's own values (each code is decoded by the same elementwise
    formula) without running the formula once per element."""
    t = _FP8_TABLES.get(kind)
    if t is None:
        t = _FP8_DECODERS[kind](np.arange(256, dtype=np.uint8))
        t.setflags(write=False)
        _FP8_TABLES[kind] = t
    return t


def to_float64(arr, kind):
    a = np.asarray(arr)
    if kind == "f32":
        assert a.dtype == np.float32, a.dtype
        return a.astype(np.float64)
    if kind == "f16":
        assert a.dtype == np.float16, a.dtype
        return a.astype(np.float64)
    if kind == "bf16":
        assert a.dtype == np.uint16, a.dtype
        bits32 = a.astype(np.uint32) << np.uint32(16)
        return bits32.view(np.float32).astype(np.float64)
    if kind in FP8_KINDS:
        assert a.dtype == np.uint8, a.dtype
        return fp8_table(kind)[a]
    raise ValueError(f"unknown storage kind {kind!r}")


def head_scales(scale, num_heads):
    """A per-tensor scale, or one scale per kv head, as float64 [num_heads]
    holding the float32 values the kernels read."""
    s = np.asarray(scale, dtype=np.float32).reshape(-1)
    if s.size == 1:
        s = np.repeat(s, num_heads)
    assert s.size == num_heads, (s.size, num_heads)
    return s.astype(np.float64)
