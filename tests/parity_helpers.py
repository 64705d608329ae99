"""Shared helpers for the GPU parity tests: run a workload's step through the
C ABI and compute the oracle's answer for the same seeded inputs."""

import sys

import numpy as np

import oracle

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3, "fp8_e4m3": 2e-2,
       "fp8_e5m2": 2e-2}


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def oracle_pools(w):
    """Pools after this step's copies and writes, per the oracle."""
    kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
    return oracle.cache_write(kp, vp, w.kv_kind, w.key, w.value, w.src_kind,
                              w.slot_mapping, w.block_size, w.k_scale,
                              w.v_scale)


def oracle_out(w, pools, rows=None):
    kp, vp = pools
    if rows is None:
        return oracle.paged_attention(w.query, w.q_kind, kp, vp, w.kv_kind,
                                      w.block_tables, w.seq_lens,
                                      w.block_size, w.scale, w.k_scale,
                                      w.v_scale)
    return oracle.paged_attention_rows(w.query, w.q_kind, kp, vp, w.kv_kind,
                                       w.block_tables, w.seq_lens,
                                       w.block_size, w.scale, rows,
                                       w.k_scale, w.v_scale)


def assert_pools_bitwise(dev, pools):
    import torch
    torch.cuda.synchronize()
    kp, vp = dev.pools_host()
    ek, ev = pools
    assert kp.tobytes() == ek.tobytes(), "k_cache differs from the oracle"
    assert vp.tobytes() == ev.tobytes(), "v_cache differs from the oracle"


def max_abs_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def check_attention(dev, w, pools, rows=None, tol=None, max_waves=0):
    import torch
    dev.attend(max_waves=max_waves)
    torch.cuda.synchronize()
    out = dev.out.cpu().numpy()
    ref = oracle_out(w, pools, rows)
    if rows is not None:
        out = np.stack([out[s, h] for s, h in rows]) if rows else out[:0, 0]
    err = max_abs_err(out, ref)
    tol = TOL[w.kv_kind] if tol is None else tol
    assert err <= tol, f"max abs error {err:.3g} > {tol}"
    return err, out
