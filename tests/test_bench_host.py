"""Host-side pieces of bench.py that run without a GPU: the CPU baseline
(the oracle timed on a bounded sample) for each scale layout, and the
algorithmic byte counts it divides by."""

import numpy as np

import bench
from paged_kv_cache_336_amd import workloads as W


def _small(kv, **kw):
    return W.custom_decode(seed=5, num_seqs=3, lens=[100, 300, 50], hq=8,
                           hkv=2, d=64, bs=16, q_kind="bf16", kv_kind=kv,
                           **kw)


def test_cpu_baseline_per_tensor_and_per_token_scales():
    for w in (_small("bf16"), _small("fp8_e4m3"),
              _small("fp8_e4m3", per_token_scales=True)):
        gbps, tok_s, sample, threads = bench.cpu_baseline(w, 0.2)
        assert gbps > 0 and tok_s > 0 and threads >= 1
        assert w.name in sample


def test_attention_bytes_count_each_live_row_once():
    w = _small("bf16")
    B = bench.algorithmic_bytes(w)["attention"]
    kv = int(np.sum(w.seq_lens)) * w.num_kv_heads * w.head_dim * 2 * 2
    q_out = w.num_seqs * w.num_q_heads * w.head_dim * (2 + 4)
    tables = int(np.sum((w.seq_lens + 15) // 16)) * 4 + 4 * w.num_seqs
    assert B == kv + q_out + tables
