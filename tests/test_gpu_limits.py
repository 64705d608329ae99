"""The largest calls the library accepts, against the oracle through the C
ABI on the GPU: paged_attn_decode with its maximum of 8192 sequences (the
per-sequence prefix then fills most of the kernel's LDS, with float32 and
bf16 operands), paged_attn_multi with its maximum of 4096 sequences, and
the one-sequence-past-the-limit calls refused before any launch."""

import numpy as np
import pytest

import oracle
from paged_kv_cache_336_amd import ops
from paged_kv_cache_336_amd import workloads as W
from paged_kv_cache_336_amd.step import DeviceStep, MultiStep

from parity_helpers import TOL, max_abs_err, oracle_pools, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("q,kv,d,hq,hkv", [("bf16", "bf16", 64, 8, 2),
                                           ("f32", "f32", 128, 4, 4)])
def test_decode_most_sequences(q, kv, d, hq, hkv):
    import torch
    say(f"decode 8192 sequences {q}/{kv} D{d}")
    lens = np.random.default_rng(41).integers(0, 48, 8192)
    w = W.custom_decode(seed=41, num_seqs=8192, lens=lens, hq=hq, hkv=hkv,
                        d=d, bs=16, q_kind=q, kv_kind=kv)
    pools = oracle_pools(w)
    dev = DeviceStep(w, replicas=False)
    dev.copy()
    dev.write()
    for waves in (0, 96):
        dev.attend(max_waves=waves)
        torch.cuda.synchronize()
        ref = oracle.paged_attention(w.query, q, pools[0], pools[1], kv,
                                     w.block_tables, w.seq_lens, 16, w.scale)
        err = max_abs_err(dev.out.cpu().numpy(), ref)
        say(f"  waves {waves}: max abs err {err:.3g}")
        assert err <= TOL[kv]


def test_multi_most_sequences():
    import torch
    say("multi-query 4096 sequences")
    rng = np.random.default_rng(42)
    lens = rng.integers(1, 40, 4096)
    qlens = np.minimum(lens, rng.integers(0, 6, 4096))
    mq = W.custom_multi(seed=42, lens=lens, qlens=qlens, hq=8, hkv=2, d=64,
                        bs=16, q_kind="bf16", kv_kind="bf16")
    dev = MultiStep(mq, replicas=False)
    dev.copy()
    dev.write()
    dev.attend()
    torch.cuda.synchronize()
    ref = oracle.paged_attention_multi(mq.query, "bf16", *oracle_pools(mq.w),
                                       "bf16", mq.w.block_tables,
                                       mq.w.seq_lens, mq.query_start, 16,
                                       mq.w.scale)
    err = max_abs_err(dev.out.cpu().numpy(), ref)
    say(f"  max abs err {err:.3g}")
    assert err <= TOL["bf16"]


def test_one_past_the_limits_is_refused():
    import torch
    lens = [3] * 8193
    w = W.custom_decode(seed=43, num_seqs=8193, lens=lens, hq=2, hkv=1, d=64,
                        bs=16, q_kind="bf16", kv_kind="bf16")
    dev = DeviceStep(w, replicas=False)
    with pytest.raises(ops.PagedKVError) as e:
        dev.attend()
    assert e.value.status == 4                       # PKV_ERR_UNSUPPORTED
    mq = W.custom_multi(seed=44, lens=[3] * 4097, qlens=[1] * 4097, hq=2,
                        hkv=1, d=64, bs=16, q_kind="bf16", kv_kind="bf16")
    md = MultiStep(mq, replicas=False)
    with pytest.raises(ops.PagedKVError) as e:
        md.attend()
    assert e.value.status == 4
    torch.cuda.synchronize()
