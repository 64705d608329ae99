"""paged_attn_decode_noalloc (no workspace argument: the library's own
device scratch) through the C ABI on the GPU, against paged_attn_decode on
the same inputs: bit for bit on two calls in a row, the second with a
smaller batch, and within the tolerance of the float64 oracle."""

import numpy as np
import pytest

from paged_kv_cache_336_amd import ops
from paged_kv_cache_336_amd import workloads as W
from paged_kv_cache_336_amd.step import DeviceStep

from parity_helpers import TOL, max_abs_err, oracle_out, oracle_pools, say

pytestmark = pytest.mark.gpu


def decode_both(w, max_waves):
    """(workspace call's output, no-alloc call's output) on the pools after
    the step's copy and write."""
    import torch
    dev = DeviceStep(w, replicas=False)
    dev.copy()
    dev.write()
    dev.attend(max_waves=max_waves)
    torch.cuda.synchronize()
    ref = dev.out.cpu().numpy().copy()
    dev.out.fill_(float("nan"))
    ops.paged_attn_decode_noalloc(
        dev.out, dev.query, dev.k_cache, dev.v_cache,
        dev.sets[0]["block_tables"], dev.seq_lens, dev.max_seq_len, w.scale,
        k_scale=dev.k_scale, v_scale=dev.v_scale, max_waves=max_waves,
        cache_kind=dev.cache_kind, kv_stream=dev.sets[0]["kv_stream"])
    torch.cuda.synchronize()
    return ref, dev.out.cpu().numpy().copy()


@pytest.mark.parametrize("max_waves", [0, 40])
def test_noalloc_matches_workspace_call(max_waves):
    """Two calls in a row on one GPU, the second with fewer and shorter
    sequences (whatever the first left in the scratch must not matter)."""
    cases = [
        W.custom_decode(seed=71, num_seqs=12,
                        lens=[1, 17, 400, 2100, 64, 0, 999, 31, 33, 700, 5,
                              1500], hq=32, hkv=8, d=128, bs=16,
                        q_kind="bf16", kv_kind="bf16"),
        W.custom_decode(seed=72, num_seqs=3, lens=[90, 2, 260], hq=32,
                        hkv=8, d=128, bs=16, q_kind="bf16", kv_kind="bf16"),
    ]
    for w in cases:
        say(f"no-alloc decode: {w.num_seqs} seqs, waves {max_waves or 'all'}")
        ref, got = decode_both(w, max_waves)
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
        err = max_abs_err(got, oracle_out(w, oracle_pools(w)))
        assert err <= TOL[w.kv_kind], err


def test_noalloc_fp8_and_limits():
    """An fp8 cache (16 query heads per kv head: the largest partial slot)
    bit for bit against the workspace call; more than 1024 waves refused."""
    import torch
    w = W.custom_decode(seed=73, num_seqs=5, lens=[3000, 40, 1, 777, 64],
                        hq=32, hkv=2, d=128, bs=32, q_kind="bf16",
                        kv_kind="fp8_e4m3")
    say("no-alloc decode: fp8, G 16")
    ref, got = decode_both(w, 0)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    dev = DeviceStep(w, replicas=False)
    with pytest.raises(ops.PagedKVError) as e:
        ops.paged_attn_decode_noalloc(
            dev.out, dev.query, dev.k_cache, dev.v_cache,
            dev.sets[0]["block_tables"], dev.seq_lens, dev.max_seq_len,
            w.scale, k_scale=dev.k_scale, v_scale=dev.v_scale,
            max_waves=1028, cache_kind=dev.cache_kind)
    assert e.value.status == 4
    torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(16))
def test_noalloc_random_shapes(seed):
    """The random decode shapes (every cache and query type pairing, G up
    to 20, both head_dims, any block size, empty sequences, per-tensor and
    per-head fp8 scales, several wave caps), one after another on the same
    scratch: bit for bit against the workspace call."""
    from dataclasses import replace
    from test_gpu_random import draw_decode
    c = draw_decode(400 + seed)
    say(f"no-alloc random {seed}: {c}")
    w = W.custom_decode(seed=4400 + seed, num_seqs=len(c["lens"]),
                        lens=c["lens"], hq=c["hq"], hkv=c["hkv"], d=c["d"],
                        bs=c["bs"], q_kind=c["q"], kv_kind=c["kv"],
                        per_head_scales=c["per_head"])
    if c["kv"].startswith("fp8"):
        w = replace(w, k_scale=np.float32(4) * w.k_scale,
                    v_scale=np.float32(4) * w.v_scale)
    ref, got = decode_both(w, c["waves"])
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
