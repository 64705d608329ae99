"""paged_attn_decode_fused (the new token's write and the attention in one
launch) against the separate calls it replaces, through the C ABI on the GPU:
the output and both pools must be identical bit for bit to cache_write_slots
followed by paged_attn_decode, for every cache type, uniform and non-uniform
block sizes, empty sequences, skipped slots, any wave split and the
full-size decode batches; small cases are also checked against the
oracle."""

import numpy as np
import pytest

from paged_kv_cache_336_amd import workloads as W
from paged_kv_cache_336_amd.step import DeviceStep, _to_torch

from parity_helpers import (TOL, assert_pools_bitwise, max_abs_err,
                            oracle_out, oracle_pools, say)

pytestmark = pytest.mark.gpu


def per_sequence_rows(w):
    """key, value [S, Hkv, D] and slots [S] for the fused call: each
    sequence's new row (the step writes one per non-empty sequence, in
    order) and slot; empty sequences get a zero row and slot -1."""
    S = w.num_seqs
    lens = w.seq_lens
    shape = (S,) + w.key.shape[1:]
    key = np.zeros(shape, dtype=w.key.dtype)
    value = np.zeros(shape, dtype=w.value.dtype)
    slots = np.full(S, -1, dtype=np.int32)
    live = np.flatnonzero(lens > 0)
    assert w.num_tokens == len(live)
    key[live] = w.key
    value[live] = w.value
    slots[live] = w.slot_mapping
    return key, value, slots


def run_pair(w, max_waves=0, drop=()):
    """(separate, fused) DeviceSteps after one step each; `drop` lists
    sequences whose slot is set to -1 (no write) in both."""
    import torch
    key, value, slots = per_sequence_rows(w)
    for s in drop:
        slots[s] = -1
    sep = DeviceStep(w, replicas=False)
    fus = DeviceStep(w, replicas=False)
    for d in (sep, fus):
        d.key = _to_torch(key, w.src_kind, "cuda")
        d.value = _to_torch(value, w.src_kind, "cuda")
        d.sets[0]["slot_mapping"] = torch.from_numpy(slots).cuda()
    sep.copy()
    sep.write()
    sep.attend(max_waves=max_waves)
    fus.copy()
    fus.attend_fused(max_waves=max_waves)
    torch.cuda.synchronize()
    return sep, fus


def assert_same(sep, fus):
    a = sep.out.cpu().numpy()
    b = fus.out.cpu().numpy()
    bad = np.argwhere(a.view(np.uint32) != b.view(np.uint32))
    assert bad.size == 0, (
        f"fused output differs from write + decode at {len(bad)} elements, "
        f"(sequence, head) pairs {sorted(set(map(tuple, bad[:, :2].tolist())))[:16]}, "
        f"max abs difference {np.max(np.abs(a.astype(np.float64) - b)):.3g}")
    ka, va = sep.pools_host()
    assert_pools_bitwise(fus, (ka, va))


SMALL = [
    # (q, kv, D, bs, hq, hkv, lens, waves)
    ("f32", "f32", 64, 4, 1, 1, [22], 0),
    ("f32", "f32", 128, 16, 4, 2, [1, 31, 32, 33, 200], 8),
    ("f32", "f32", 64, 3, 8, 8, [5, 97], 4),
    ("bf16", "bf16", 128, 16, 32, 8, [1, 2, 15, 16, 17, 300, 3000], 0),
    ("bf16", "bf16", 128, 1, 4, 4, [1, 40, 70], 4),
    ("bf16", "bf16", 64, 48, 12, 2, [47, 48, 49, 500], 12),
    ("bf16", "bf16", 128, 544, 8, 1, [543, 544, 545, 2000], 8),
    ("f16", "f16", 128, 16, 64, 8, [1, 100, 1023, 4100], 16),
    ("f16", "f16", 64, 5, 20, 2, [9, 64, 130], 4),
    ("bf16", "fp8_e4m3", 128, 64, 32, 8, [1, 63, 64, 65, 9000], 4),
    ("bf16", "fp8_e4m3", 64, 4, 4, 2, [3, 90], 0),
    ("f16", "fp8_e4m3", 128, 16, 8, 8, [17, 600], 8),
    ("f32", "fp8_e4m3", 64, 16, 2, 1, [1, 33, 300], 8),
    ("bf16", "bf16", 128, 16, 8, 8, [0, 5, 0, 40], 4),
    ("bf16", "fp8_e5m2", 128, 16, 16, 4, [3, 700, 65], 4),
    ("f32", "fp8_e5m2", 64, 32, 4, 2, [100, 33], 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[
    f"{c[0]}-{c[1]}-D{c[2]}-bs{c[3]}-G{c[4] // c[5]}-L{max(c[6])}-W{c[7]}"
    for c in SMALL])
def test_fused_small(case):
    q, kv, d, bs, hq, hkv, lens, waves = case
    say(f"fused small {case}")
    w = W.custom_decode(seed=500 + SMALL.index(case), num_seqs=len(lens),
                        lens=lens, hq=hq, hkv=hkv, d=d, bs=bs, q_kind=q,
                        kv_kind=kv)
    # the whole grid: one fused launch; a few waves: with more rows than
    # waves the write goes as its own launch first
    for wv in (0, waves) if waves else (0,):
        sep, fus = run_pair(w, max_waves=wv)
        assert_same(sep, fus)
        assert_pools_bitwise(fus, oracle_pools(w))
        err = max_abs_err(fus.out.cpu().numpy(),
                          oracle_out(w, oracle_pools(w)))
        assert err <= TOL[kv], f"waves {wv}: {err:.3g}"


def test_fused_skipped_slots():
    """A negative slot writes nothing: the attention then reads the position
    as the pool holds it, exactly as after a write that skipped it."""
    w = W.custom_decode(seed=531, num_seqs=5, lens=[40, 17, 300, 2, 65],
                        hq=16, hkv=4, d=128, bs=16, q_kind="bf16",
                        kv_kind="bf16")
    sep, fus = run_pair(w, drop=(1, 3))
    assert_same(sep, fus)


@pytest.mark.parametrize("name", ["llama8b_decode", "llama70b_decode",
                                  "prefix_sharing_fork_bs544",
                                  "long_context_fp8"])
def test_fused_full_size(name):
    say(f"fused full {name}")
    w = W.workload_by_name(name)
    sep, fus = run_pair(w)
    assert_same(sep, fus)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "fp8_e5m2"])
def test_fused_per_head_scales(kv):
    """The fused write encodes each head over its own scale."""
    w = W.custom_decode(seed=532, num_seqs=4, lens=[40, 300, 2, 65], hq=16,
                        hkv=4, d=128, bs=16, q_kind="bf16", kv_kind=kv,
                        per_head_scales=True)
    for wv in (0, 4):
        say(f"per-head scales {kv}: waves {wv or 'all'}")
        sep, fus = run_pair(w, max_waves=wv)
        assert_same(sep, fus)
        assert_pools_bitwise(fus, oracle_pools(w))

