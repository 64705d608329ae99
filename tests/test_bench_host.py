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


def test_default_line_runs_the_largest_16bit_decode_batch():
    """With no flags the line measures the 70B-shaped batch (256 sequences,
    1.7 GB of K/V per call); the other decode workloads it also times are
    names the generator knows."""
    import subprocess
    import sys
    src = open(bench.__file__).read()
    assert 'ap.add_argument("--workload", default="llama70b_decode"' in src
    start = src.index('ap.add_argument("--also", default="') + \
        len('ap.add_argument("--also", default="')
    also = src[start:src.index('"', start)].split(",")
    assert also and all(n in W.DECODE_WORKLOADS for n in also)
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
