"""ctypes binding of libpagedkv.so (declared in include/pagedkv.h).

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the shared library is missing the
first call raises.

Functions keep the C names: :func:`cache_write_slots`,
:func:`cache_write_slots_token_scaled`, :func:`copy_blocks`,
:func:`copy_block_prefixes`, :func:`copy_token_scales`,
:func:`copy_token_scale_prefixes`, :func:`paged_attn_decode`,
:func:`paged_attn_decode_noalloc`, :func:`paged_attn_decode_fused`,
:func:`paged_attn_workspace_size`, :func:`paged_attn_multi`,
:func:`paged_attn_multi_workspace_size`, :func:`pkv_status_string`,
:func:`pkv_set_debug_checks`.

Each operation also takes ``prepare=True``, which returns the call with its
arguments marshalled (a :class:`PreparedCall`) instead of making it: a
serving loop whose tensors stay in place issues each step's calls again
without any per-call lookups.
"""

import collections
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3, PKV_FP8_E5M2 = 0, 1, 2, 3, 4
PKV_SCALE_PER_HEAD = 0x100
PKV_SCALE_PER_TOKEN = 0x200
PKV_KV_STREAM = 0x400       # hint: no block is read by two sequences
KIND_CODES = {"f32": PKV_F32, "f16": PKV_F16, "bf16": PKV_BF16,
              "fp8_e4m3": PKV_FP8_E4M3, "fp8_e5m2": PKV_FP8_E5M2}

EXPORTED = ("pkv_status_string", "pkv_set_debug_checks", "cache_write_slots",
            "cache_write_slots_token_scaled", "copy_blocks",
            "copy_block_prefixes", "copy_token_scales",
            "copy_token_scale_prefixes", "paged_attn_workspace_size",
            "copy_blocks_layers", "copy_block_prefixes_layers",
            "paged_attn_decode", "paged_attn_decode_noalloc",
            "paged_attn_decode_fused",
            "paged_attn_multi_workspace_size", "paged_attn_multi")

_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: status {status} "
                         f"({pkv_status_string(status)})")
        self.status = status


def load_library(path=None):
    """Load and type the library once; raise if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m paged_kv_cache_336_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    ci = ctypes.c_int
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [ci]
    lib.pkv_set_debug_checks.restype = ci
    lib.pkv_set_debug_checks.argtypes = [ci]
    lib.cache_write_slots.restype = ci
    lib.cache_write_slots.argtypes = [vp, vp, ci, vp, vp, ci, vp, i64, i64, i32,
                                      i32, i32, vp, vp, vp]
    lib.cache_write_slots_token_scaled.restype = ci
    lib.cache_write_slots_token_scaled.argtypes = [vp, vp, ci, vp, vp, ci, vp,
                                                   vp, vp, i64, i64, i32, i32,
                                                   i32, vp]
    for fn in (lib.copy_token_scales, lib.copy_token_scale_prefixes):
        fn.restype = ci
        fn.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp]
    lib.copy_blocks.restype = ci
    lib.copy_blocks.argtypes = [vp, vp, ci, vp, i64, i64, i32, i32, i32, vp]
    lib.copy_block_prefixes.restype = ci
    lib.copy_block_prefixes.argtypes = [vp, vp, ci, vp, i64, i64, i32, i32,
                                        i32, vp]
    for fn in (lib.copy_blocks_layers, lib.copy_block_prefixes_layers):
        fn.restype = ci
        fn.argtypes = [vp, vp, i64, i32, ci, vp, i64, i64, i32, i32, i32, vp]
    lib.paged_attn_workspace_size.restype = sz
    lib.paged_attn_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.paged_attn_decode.restype = ci
    lib.paged_attn_decode.argtypes = [vp, vp, ci, vp, vp, ci, vp, vp, vp, i32,
                                      vp, i32, i32, i32, i32, i32, i64, i32,
                                      f32, i32, vp, sz, vp]
    lib.paged_attn_decode_noalloc.restype = ci
    lib.paged_attn_decode_noalloc.argtypes = [vp, vp, ci, vp, vp, ci, vp, vp,
                                              vp, i32, vp, i32, i32, i32, i32,
                                              i32, i64, i32, f32, i32, vp]
    lib.paged_attn_decode_fused.restype = ci
    lib.paged_attn_decode_fused.argtypes = [vp, vp, ci, vp, vp, vp, vp, ci,
                                            vp, vp, vp, vp, i32, vp, i32, i32,
                                            i32, i32, i32, i64, i32, f32, i32,
                                            vp, sz, vp]
    lib.paged_attn_multi_workspace_size.restype = sz
    lib.paged_attn_multi_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.paged_attn_multi.restype = ci
    lib.paged_attn_multi.argtypes = [vp, vp, ci, vp, vp, ci, vp, vp, vp, i32,
                                     vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     i64, i32, f32, i32, vp, sz, vp]
    if path == LIB_PATH:
        _lib = lib
    return lib


def pkv_status_string(status):
    return load_library().pkv_status_string(int(status)).decode()


def pkv_set_debug_checks(enable):
    """Turn the library's checks of device contents on or off (see
    pagedkv.h); returns the previous setting as a bool."""
    return bool(load_library().pkv_set_debug_checks(1 if enable else 0))


# ----------------------------------------------------------------------------
# torch marshalling helpers
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t, kind=None):
    """pkv dtype of a tensor; uint8 tensors need kind='fp8_e4m3' or
    'fp8_e5m2'."""
    if kind is not None:
        return KIND_CODES[kind]
    torch = _torch()
    table = {torch.float32: PKV_F32, torch.float16: PKV_F16,
             torch.bfloat16: PKV_BF16}
    if t.dtype in table:
        return table[t.dtype]
    if t.dtype == getattr(torch, "float8_e4m3fn", None):
        return PKV_FP8_E4M3
    if t.dtype == getattr(torch, "float8_e5m2", None):
        return PKV_FP8_E5M2
    raise TypeError(f"no pkv dtype for {t.dtype}; pass kind=")


def cache_code(k_cache, cache_kind, k_scale, kv_stream=False):
    """The cache dtype argument: the element type, with PKV_SCALE_PER_TOKEN
    when an fp8 cache's scales are [num_blocks, block_size, Hkv] arrays, or
    PKV_SCALE_PER_HEAD when they hold one value per kv head; PKV_KV_STREAM
    when kv_stream is true."""
    code = dtype_code(k_cache, cache_kind)
    if code in (PKV_FP8_E4M3, PKV_FP8_E5M2) and k_scale is not None:
        if k_scale.dim() == 3:
            code |= PKV_SCALE_PER_TOKEN
        elif k_scale.numel() > 1:
            code |= PKV_SCALE_PER_HEAD
    if kv_stream:
        code |= PKV_KV_STREAM
    return code


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, t):
    """The HIP stream a call is queued on, as an integer handle: ``stream``
    if given, else the current stream of tensor t's device (read without
    building a torch Stream object, which costs microseconds per call)."""
    if stream is not None:
        return int(stream.cuda_stream)
    torch = _torch()
    idx = t.device.index
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None and idx is not None:
        return raw(idx)
    return int(torch.cuda.current_stream(t.device).cuda_stream)


def _stream(stream, t):
    return ctypes.c_void_p(_stream_handle(stream, t))


def _check(fn, status):
    if status != 0:
        raise PagedKVError(fn, status)


class PreparedCall:
    """One library call with its arguments marshalled once: pointers,
    sizes, dtype codes, the stream and, for attention, the workspace.
    Calling it issues the same call again, which is the cheapest way to
    queue a step whose buffers stay in place (a serving loop's persistent
    tensors): no shape, dtype or stream lookups per call.  The tensors it
    was made from must stay alive and in place; their contents may change
    between calls.  The ``prepare=True`` argument of the operations below
    returns one instead of making the call."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name, fn, args, keep=()):
        self.name = name
        self.fn = fn
        self.args = args
        # the workspace buffer it points at (a default workspace may be
        # replaced by a larger one later; this reference keeps the buffer
        # this call uses alive)
        self.keep = keep

    def __call__(self):
        status = self.fn(*self.args)
        if status != 0:
            raise PagedKVError(self.name, status)


def _run(name, fn, args, prepare, keep=()):
    """Make the call, or with prepare return it as a PreparedCall (holding
    `keep`, the buffers the library owns that the call points at)."""
    if prepare:
        return PreparedCall(name, fn, args, keep)
    _check(name, fn(*args))
    return None


# ----------------------------------------------------------------------------
# the three operations
# ----------------------------------------------------------------------------

def cache_write_slots(key, value, k_cache, v_cache, slot_mapping,
                      k_scale=None, v_scale=None, cache_kind=None,
                      stream=None, prepare=False):
    """Scatter key/value [T, Hkv, D] into the pools at slot_mapping (in
    place)."""
    lib = load_library()
    nb, bs, hkv, d = k_cache.shape
    return _run("cache_write_slots", lib.cache_write_slots, (
        _ptr(key), _ptr(value), dtype_code(key), _ptr(k_cache), _ptr(v_cache),
        cache_code(k_cache, cache_kind, k_scale), _ptr(slot_mapping),
        int(slot_mapping.shape[0]), nb, bs, hkv, d, _ptr(k_scale),
        _ptr(v_scale), _stream(stream, k_cache)), prepare)


def cache_write_slots_token_scaled(key, value, k_cache, v_cache, k_scales,
                                   v_scales, slot_mapping, cache_kind=None,
                                   stream=None, prepare=False):
    """Scatter key/value [T, Hkv, D] into an fp8 cache with a scale per
    written row, stored in k_scales / v_scales [num_blocks, block_size,
    Hkv] (float32, in place)."""
    lib = load_library()
    nb, bs, hkv, d = k_cache.shape
    assert tuple(k_scales.shape) == (nb, bs, hkv) and \
        tuple(v_scales.shape) == (nb, bs, hkv)
    return _run("cache_write_slots_token_scaled",
                lib.cache_write_slots_token_scaled, (
                    _ptr(key), _ptr(value), dtype_code(key), _ptr(k_cache),
                    _ptr(v_cache), dtype_code(k_cache, cache_kind) |
                    PKV_SCALE_PER_TOKEN, _ptr(k_scales), _ptr(v_scales),
                    _ptr(slot_mapping), int(slot_mapping.shape[0]), nb, bs,
                    hkv, d, _stream(stream, k_cache)), prepare)


def _scales_copy(name, k_scales, v_scales, rows, width, stream,
                 prepare=False):
    lib = load_library()
    nb, bs, hkv = k_scales.shape
    assert tuple(v_scales.shape) == (nb, bs, hkv)
    assert rows.shape[1:] == (width,)
    return _run(name, getattr(lib, name), (
        _ptr(k_scales), _ptr(v_scales), _ptr(rows), int(rows.shape[0]), nb,
        bs, hkv, _stream(stream, k_scales)), prepare)


def copy_token_scales(k_scales, v_scales, block_pairs, stream=None,
                      prepare=False):
    """Per-token scale arrays through whole-block copies [P, 2]."""
    return _scales_copy("copy_token_scales", k_scales, v_scales,
                        block_pairs, 2, stream, prepare)


def copy_token_scale_prefixes(k_scales, v_scales, block_triples,
                              stream=None, prepare=False):
    """Per-token scale arrays through token-prefix copies [P, 3]."""
    return _scales_copy("copy_token_scale_prefixes", k_scales, v_scales,
                        block_triples, 3, stream, prepare)


def copy_blocks(k_cache, v_cache, block_pairs, cache_kind=None, stream=None,
                prepare=False):
    """Copy whole blocks src -> dst for every row of block_pairs [P, 2]."""
    lib = load_library()
    nb, bs, hkv, d = k_cache.shape
    return _run("copy_blocks", lib.copy_blocks, (
        _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache, cache_kind),
        _ptr(block_pairs), int(block_pairs.shape[0]), nb, bs, hkv, d,
        _stream(stream, k_cache)), prepare)


def copy_block_prefixes(k_cache, v_cache, block_triples, cache_kind=None,
                        stream=None, prepare=False):
    """Copy the first `tokens` slots of block src to block dst for every
    row {src, dst, tokens} of block_triples [P, 3]."""
    lib = load_library()
    nb, bs, hkv, d = k_cache.shape
    return _run("copy_block_prefixes", lib.copy_block_prefixes, (
        _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache, cache_kind),
        _ptr(block_triples), int(block_triples.shape[0]), nb, bs, hkv, d,
        _stream(stream, k_cache)), prepare)


def _layers_copy(fn, k_caches, v_caches, rows, cache_kind, stream, width,
                 prepare=False):
    """k_caches, v_caches: [num_layers, num_blocks, block_size, Hkv, D]."""
    lib = load_library()
    nl, nb, bs, hkv, d = k_caches.shape
    stride = k_caches.stride(0) * k_caches.element_size()
    assert v_caches.shape == k_caches.shape and \
        v_caches.stride(0) == k_caches.stride(0)
    assert rows.shape[1:] == (width,)
    return _run(fn.__name__, fn, (
        _ptr(k_caches), _ptr(v_caches), stride, nl,
        dtype_code(k_caches, cache_kind), _ptr(rows), int(rows.shape[0]), nb,
        bs, hkv, d, _stream(stream, k_caches)), prepare)


def copy_blocks_layers(k_caches, v_caches, block_pairs, cache_kind=None,
                       stream=None, prepare=False):
    """Whole-block copies src -> dst in every layer's pools (one launch)."""
    return _layers_copy(load_library().copy_blocks_layers, k_caches,
                        v_caches, block_pairs, cache_kind, stream, 2, prepare)


def copy_block_prefixes_layers(k_caches, v_caches, block_triples,
                               cache_kind=None, stream=None, prepare=False):
    """copy_block_prefixes in every layer's pools (one launch)."""
    return _layers_copy(load_library().copy_block_prefixes_layers, k_caches,
                        v_caches, block_triples, cache_kind, stream, 3,
                        prepare)


def paged_attn_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim):
    v = load_library().paged_attn_workspace_size(num_seqs, num_q_heads,
                                                 num_kv_heads, head_dim)
    if v == ctypes.c_size_t(-1).value:
        raise PagedKVError("paged_attn_workspace_size", 2)
    return v


def paged_attn_multi_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                    head_dim):
    v = load_library().paged_attn_multi_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim)
    if v == ctypes.c_size_t(-1).value:
        raise PagedKVError("paged_attn_multi_workspace_size", 2)
    return v


class Workspace:
    """A device workspace for the attention calls, grown (never shrunk) to
    the largest size asked for; it needs no initialisation.

    A workspace serves one stream: two calls that share it must not
    overlap in time, which calls on one stream never do.  It is allocated
    while ``stream`` is current, so torch's caching allocator ties the
    memory to the stream the kernels use it on, and a buffer dropped when
    the workspace grows is reused only after the work queued on that stream
    before the drop (torch's stream-ordered reuse)."""

    def __init__(self, device="cuda", stream=None):
        self.device = device
        self.stream = stream
        self.buf = None

    def get(self, nbytes):
        torch = _torch()
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = None
            if self.stream is not None:
                with torch.cuda.stream(self.stream):
                    self.buf = torch.empty(int(nbytes), dtype=torch.uint8,
                                           device=self.device)
            else:
                self.buf = torch.empty(int(nbytes), dtype=torch.uint8,
                                       device=self.device)
        return self.buf


# default workspaces, one per (device, stream): calls on different streams
# never share one (they could overlap in time).  The most recently used
# _DEFAULT_WS_KEEP are kept; dropping one is safe, as its buffer was
# allocated on its own stream and torch reuses it only in that stream's order
# (and a prepared call holds the buffer it was made with).
_default_ws = collections.OrderedDict()
_DEFAULT_WS_KEEP = 16
_NO_SIZE = (1 << 64) - 1     # (size_t)-1: the size query's "invalid"


def _default_workspace(device, stream, handle):
    """The default workspace of (device, stream handle); created while that
    stream is current (``stream`` None: it is the current stream)."""
    key = (device.index, handle)
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(device, stream)
        while len(_default_ws) > _DEFAULT_WS_KEEP:
            _default_ws.popitem(last=False)
    else:
        _default_ws.move_to_end(key)
    return ws


def _workspace_buf(workspace, need):
    """The buffer to pass: none for a shape the size query calls invalid
    (the call itself then reports why), else the caller's buffer or a
    Workspace grown to the size."""
    if need == _NO_SIZE:
        return None
    return workspace.get(need) if isinstance(workspace, Workspace) \
        else workspace


def paged_attn_decode(out, query, k_cache, v_cache, block_tables, seq_lens,
                      max_seq_len, scale, k_scale=None, v_scale=None,
                      max_waves=0, workspace=None, cache_kind=None,
                      stream=None, kv_stream=False, prepare=False):
    """out[S, Hq, D] (float32) = paged decode attention; see pagedkv.h.
    kv_stream=True passes PKV_KV_STREAM (no block read by two sequences)."""
    lib = load_library()
    s, hq, d = query.shape
    nb, bs, hkv, _ = k_cache.shape
    need = lib.paged_attn_workspace_size(s, hq, hkv, d)
    handle = _stream_handle(stream, query)
    if workspace is None:
        workspace = _default_workspace(query.device, stream, handle)
    buf = _workspace_buf(workspace, need)
    return _run("paged_attn_decode", lib.paged_attn_decode, (
        _ptr(out), _ptr(query), dtype_code(query), _ptr(k_cache),
        _ptr(v_cache), cache_code(k_cache, cache_kind, k_scale, kv_stream),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
        int(block_tables.shape[1]),
        _ptr(seq_lens), int(max_seq_len), s, hq, hkv, d, nb, bs, float(scale),
        int(max_waves), _ptr(buf),
        0 if buf is None else buf.numel() * buf.element_size(),
        ctypes.c_void_p(handle)), prepare, (buf,))


def paged_attn_decode_noalloc(out, query, k_cache, v_cache, block_tables,
                              seq_lens, max_seq_len, scale, k_scale=None,
                              v_scale=None, max_waves=0, cache_kind=None,
                              stream=None, kv_stream=False, prepare=False):
    """paged_attn_decode with the library's own scratch instead of a
    workspace: allocates nothing (see pagedkv.h)."""
    lib = load_library()
    s, hq, d = query.shape
    nb, bs, hkv, _ = k_cache.shape
    return _run("paged_attn_decode_noalloc", lib.paged_attn_decode_noalloc, (
        _ptr(out), _ptr(query), dtype_code(query), _ptr(k_cache),
        _ptr(v_cache), cache_code(k_cache, cache_kind, k_scale, kv_stream),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), s, hq,
        hkv, d, nb, bs, float(scale), int(max_waves),
        _stream(stream, query)), prepare)


def paged_attn_decode_fused(out, query, key, value, k_cache, v_cache,
                            slot_mapping, block_tables, seq_lens, max_seq_len,
                            scale, k_scale=None, v_scale=None, max_waves=0,
                            workspace=None, cache_kind=None, stream=None,
                            kv_stream=False, prepare=False):
    """cache_write_slots of one new token per sequence fused into
    paged_attn_decode; see pagedkv.h (kv_stream as for paged_attn_decode)."""
    lib = load_library()
    s, hq, d = query.shape
    nb, bs, hkv, _ = k_cache.shape
    need = lib.paged_attn_workspace_size(s, hq, hkv, d)
    handle = _stream_handle(stream, query)
    if workspace is None:
        workspace = _default_workspace(query.device, stream, handle)
    buf = _workspace_buf(workspace, need)
    return _run("paged_attn_decode_fused", lib.paged_attn_decode_fused, (
        _ptr(out), _ptr(query), dtype_code(query), _ptr(key), _ptr(value),
        _ptr(k_cache), _ptr(v_cache),
        cache_code(k_cache, cache_kind, k_scale, kv_stream),
        _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), s, hq,
        hkv, d, nb, bs, float(scale), int(max_waves), _ptr(buf),
        0 if buf is None else buf.numel() * buf.element_size(),
        ctypes.c_void_p(handle)), prepare, (buf,))


def paged_attn_multi(out, query, k_cache, v_cache, block_tables, seq_lens,
                     query_start, max_query_len, max_seq_len, scale,
                     k_scale=None, v_scale=None, max_waves=0, workspace=None,
                     cache_kind=None, stream=None, kv_stream=False,
                     prepare=False):
    """out[T, Hq, D] (float32) = paged attention of T new query tokens,
    causal among each sequence's new tokens; see pagedkv.h (kv_stream as
    for paged_attn_decode)."""
    lib = load_library()
    t, hq, d = query.shape
    nb, bs, hkv, _ = k_cache.shape
    s = int(seq_lens.shape[0])
    need = lib.paged_attn_multi_workspace_size(s, hq, hkv, d)
    handle = _stream_handle(stream, query)
    if workspace is None:
        workspace = _default_workspace(query.device, stream, handle)
    buf = _workspace_buf(workspace, need)
    return _run("paged_attn_multi", lib.paged_attn_multi, (
        _ptr(out), _ptr(query), dtype_code(query), _ptr(k_cache),
        _ptr(v_cache), cache_code(k_cache, cache_kind, k_scale, kv_stream),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
        int(block_tables.shape[1]),
        _ptr(seq_lens), _ptr(query_start), t, int(max_query_len),
        int(max_seq_len), s, hq, hkv, d, nb, bs, float(scale),
        int(max_waves), _ptr(buf),
        0 if buf is None else buf.numel() * buf.element_size(),
        ctypes.c_void_p(handle)), prepare, (buf,))
