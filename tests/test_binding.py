"""The Python binding on the host (CPU only, no compute call): a prepared
call holds the marshalled arguments and makes the library call only when it
is called, reporting the status the same way as a direct call, and keeps
the workspace buffer it points at alive; the default workspaces (one per
device and stream) are bounded to the most recently used."""

import ctypes

import pytest
import torch

from paged_kv_cache_336_amd import ops


class _FakeStream:
    cuda_stream = 0


def _decode_args():
    # float16 query over a bfloat16 cache: rejected by the host checks
    # before any HIP call (PKV_ERR_DTYPE)
    q = torch.zeros(2, 8, 128, dtype=torch.float16)
    kc = torch.zeros(4, 16, 2, 128, dtype=torch.bfloat16)
    out = torch.zeros(2, 8, 128, dtype=torch.float32)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    sl = torch.ones(2, dtype=torch.int32)
    return out, q, kc, bt, sl


def test_prepared_call_defers_and_reports_status():
    out, q, kc, bt, sl = _decode_args()
    ws = torch.empty(ops.paged_attn_workspace_size(2, 8, 2, 128),
                     dtype=torch.uint8)
    call = ops.paged_attn_decode(out, q, kc, kc, bt, sl, 64, 0.1,
                                 workspace=ws, stream=_FakeStream(),
                                 prepare=True)
    assert isinstance(call, ops.PreparedCall)
    assert call.name == "paged_attn_decode"
    assert call.args[-1].value in (None, 0)      # the stream handle given
    with pytest.raises(ops.PagedKVError) as e:
        call()
    assert e.value.status == 3
    with pytest.raises(ops.PagedKVError) as e2:   # direct call: same status
        ops.paged_attn_decode(out, q, kc, kc, bt, sl, 64, 0.1, workspace=ws,
                              stream=_FakeStream())
    assert e2.value.status == 3


def test_prepared_copy_with_nothing_to_copy_succeeds():
    kc = torch.zeros(4, 16, 2, 128, dtype=torch.float16)
    pairs = torch.zeros(0, 2, dtype=torch.int32)
    call = ops.copy_blocks(kc, kc, pairs, stream=_FakeStream(), prepare=True)
    assert isinstance(call, ops.PreparedCall)
    call()                                         # zero pairs: status 0
    assert isinstance(call.args[-1], ctypes.c_void_p)


def test_prepared_call_keeps_its_workspace_buffer():
    # a Workspace replaces its buffer when it grows; the prepared call keeps
    # the buffer its marshalled pointer names alive
    out, q, kc, bt, sl = _decode_args()
    ws = ops.Workspace("cpu")
    call = ops.paged_attn_decode(out, q, kc, kc, bt, sl, 64, 0.1,
                                 workspace=ws, stream=_FakeStream(),
                                 prepare=True)
    (held,) = call.keep
    first = held.data_ptr()
    ws.get(held.numel() * 4)                     # grows: a new buffer
    assert ws.buf is not held
    assert call.keep[0] is held and held.data_ptr() == first
    ptr = call.args[-3]
    assert (ptr.value if isinstance(ptr, ctypes.c_void_p) else ptr) == first


def test_default_workspaces_are_bounded():
    # one default workspace per (device, stream) in use, the most recently
    # used kept
    ops._default_ws.clear()
    dev = torch.device("cpu")
    first = ops._default_workspace(dev, None, 1000)
    for h in range(1001, 1001 + ops._DEFAULT_WS_KEEP + 5):
        ops._default_workspace(dev, None, h)
    assert len(ops._default_ws) == ops._DEFAULT_WS_KEEP
    assert (None, 1000) not in ops._default_ws
    again = ops._default_workspace(dev, None, 1000)
    assert again is not first
    last = ops._default_workspace(dev, None, 1001 + ops._DEFAULT_WS_KEEP + 4)
    assert ops._default_workspace(dev, None,
                                  1001 + ops._DEFAULT_WS_KEEP + 4) is last
    ops._default_ws.clear()
