"""Pins for the oracle's slot-mapped write and block copy (CPU only).

* The worked example's slot list (page 2's figure) scatters 22 tokens so that
  walking the table [7, 2, 11, 5, 9, 0] reads them back in order, and no
  block outside the table changes.
* The page-1 code example (64 blocks, block size 32, 8 heads, D 128, fp16,
  slot_mapping = arange(4)) lands tokens 0..3 in block 0 at offsets 0..3 and
  leaves every other byte alone.
* An fp8 cache stores torch's float8_e4m3fn cast of float32(x)/float32(scale)
  (library routine) for in-range values, at a power-of-two and a
  non-power-of-two scale.
* Block copies make destinations equal to sources bit for bit.
"""

import json
import os

import numpy as np
import torch

import oracle
from oracle import cache_write, copy_blocks, gather_sequence


def test_worked_example_scatter(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    bs, L, nb, d = g["block_size"], g["seq_len"], 16, 64
    rng = np.random.default_rng(0)
    kp = np.full((nb, bs, 1, d), np.nan, dtype=np.float32)
    others = [b for b in range(nb) if b not in g["physical_blocks"]]
    kp[others] = rng.standard_normal((len(others), bs, 1, d))
    vp = kp.copy()
    key = rng.standard_normal((L, 1, d)).astype(np.float32)
    val = rng.standard_normal((L, 1, d)).astype(np.float32)
    k2, v2 = cache_write(kp, vp, "f32", key, val, "f32",
                         np.array(g["slot_mapping"], dtype=np.int32), bs)
    table = np.array(g["physical_blocks"], dtype=np.int32)
    assert np.array_equal(gather_sequence(k2, table, L, bs, 0), key[:, 0])
    assert np.array_equal(gather_sequence(v2, table, L, bs, 0), val[:, 0])
    assert np.array_equal(k2[others], kp[others])
    # the last block keeps its 2 unused slots untouched (poison stays)
    assert np.isnan(k2[g["physical_blocks"][-1], L % bs:]).all()
    assert bs * len(table) - L == g["wasted_slots_in_last_block"]


def test_page_one_write_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "write_example.json")))
    nb, bs, h, d = g["num_blocks"], g["block_size"], g["num_kv_heads"], \
        g["head_dim"]
    rng = np.random.default_rng(1)
    kp = rng.standard_normal((nb, bs, h, d)).astype(np.float16)
    vp = rng.standard_normal((nb, bs, h, d)).astype(np.float16)
    key = rng.standard_normal((4, h, d)).astype(np.float16)
    val = rng.standard_normal((4, h, d)).astype(np.float16)
    slots = np.array(g["slot_mapping"], dtype=np.int32)
    k2, v2 = cache_write(kp, vp, "f16", key, val, "f16", slots, bs)
    for t in range(4):
        assert k2[0, t].tobytes() == key[t].tobytes()
        assert v2[0, t].tobytes() == val[t].tobytes()
    mask = np.ones((nb, bs), dtype=bool)
    mask[0, :4] = False
    assert k2[mask].tobytes() == kp[mask].tobytes()
    assert v2[mask].tobytes() == vp[mask].tobytes()


def test_negative_slots_are_skipped():
    rng = np.random.default_rng(2)
    kp = rng.standard_normal((4, 4, 2, 8)).astype(np.float32)
    vp = kp.copy()
    key = rng.standard_normal((3, 2, 8)).astype(np.float32)
    k2, v2 = cache_write(kp, vp, "f32", key, key, "f32",
                         np.array([-1, 5, -7], dtype=np.int32), 4)
    assert np.array_equal(k2[1, 1], key[1])
    k2[1, 1] = kp[1, 1]
    assert np.array_equal(k2, kp)


def _torch_e4m3(x32):
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_fp8_write_matches_torch_cast():
    rng = np.random.default_rng(3)
    T, h, d, bs, nb = 12, 2, 64, 8, 5
    key = rng.standard_normal((T, h, d)).astype(np.float32)
    val = (rng.standard_normal((T, h, d)) * 3).astype(np.float32)
    # as bf16 source rows (the workloads' source dtype for fp8 caches)
    kb = torch.from_numpy(key).to(torch.bfloat16)
    vb = torch.from_numpy(val).to(torch.bfloat16)
    key_bits = kb.view(torch.int16).numpy().view(np.uint16)
    val_bits = vb.view(torch.int16).numpy().view(np.uint16)
    slots = rng.permutation(nb * bs)[:T].astype(np.int32)
    pool = np.zeros((nb, bs, h, d), dtype=np.uint8)
    for k_scale, v_scale in ((1.0, 0.25), (0.0123, 0.0371)):
        k2, v2 = cache_write(pool, pool, "fp8_e4m3", key_bits, val_bits,
                             "bf16", slots, bs, k_scale, v_scale)
        ks = np.float32(k_scale)
        vs = np.float32(v_scale)
        exp_k = kb.float().numpy() / ks
        exp_v = vb.float().numpy() / vs
        in_range = (np.abs(exp_k) <= 448).all() and (np.abs(exp_v) <= 448).all()
        for t in range(T):
            b, o = divmod(int(slots[t]), bs)
            if np.abs(exp_k[t]).max() <= 448:
                assert np.array_equal(k2[b, o], _torch_e4m3(exp_k[t]))
            if np.abs(exp_v[t]).max() <= 448:
                assert np.array_equal(v2[b, o], _torch_e4m3(exp_v[t]))
        if not in_range:
            # out-of-range elements saturate to the largest magnitude
            sat = np.abs(exp_k) > 464
            if sat.any():
                vals = np.stack([k2[divmod(int(s), bs)] for s in slots])
                assert ((vals[sat] & 0x7F) == 0x7E).all()


def test_copy_blocks_bitwise():
    rng = np.random.default_rng(4)
    kp = rng.standard_normal((10, 6, 2, 4)).astype(np.float16)
    vp = rng.standard_normal((10, 6, 2, 4)).astype(np.float16)
    pairs = np.array([[3, 7], [1, 0], [9, 2]], dtype=np.int32)
    k2, v2 = copy_blocks(kp, vp, pairs)
    for src, dst in pairs:
        assert k2[dst].tobytes() == kp[src].tobytes()
        assert v2[dst].tobytes() == vp[src].tobytes()
    untouched = [b for b in range(10) if b not in pairs[:, 1]]
    assert k2[untouched].tobytes() == kp[untouched].tobytes()
    k3, v3 = copy_blocks(kp, vp, np.zeros((0, 2), dtype=np.int32))
    assert k3.tobytes() == kp.tobytes() and v3.tobytes() == vp.tobytes()


def test_copy_of_the_tokens_a_block_holds():
    # the FAQ entry on copy-on-write: the existing tokens go into the new
    # block; slots past them are not copied
    rng = np.random.default_rng(3)
    kp = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    vp = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    k2, v2 = oracle.copy_block_prefixes(kp, vp, [[1, 4, 3], [2, 5, 0]])
    assert np.array_equal(k2[4, :3], kp[1, :3]) and np.array_equal(k2[4, 3], kp[4, 3])
    assert np.array_equal(v2[4, :3], vp[1, :3]) and np.array_equal(v2[4, 3], vp[4, 3])
    assert np.array_equal(k2[5], kp[5]) and np.array_equal(v2[5], vp[5])
    untouched = [0, 1, 2, 3]
    assert np.array_equal(k2[untouched], kp[untouched])
    # a count of a whole block (or more) is the whole-block copy
    kw, vw = oracle.copy_blocks(kp, vp, [[1, 4]])
    kf, vf = oracle.copy_block_prefixes(kp, vp, [[1, 4, 4]])
    kc, vc = oracle.copy_block_prefixes(kp, vp, [[1, 4, 9]])
    assert np.array_equal(kw, kf) and np.array_equal(kw, kc)
    assert np.array_equal(vw, vf) and np.array_equal(vw, vc)
