"""Seeded random shapes through the decode and multi-query calls, through the
C ABI on the GPU, against the float64 oracle.  Each case draws its cache and
query types, the heads and their grouping (G up to 20 for decode, where rows
of more than 16 query heads are cut into chunks), head_dim, block size
(multiples of 16 and not), the lengths (empty sequences, lengths on and off
block and tile boundaries), fp8 scales per tensor or per kv head, and the
wave cap, so the combinations the hand-picked cases do not name are run too.
The step's copy and write go first, as in every parity test, and the pools
they leave must equal the oracle's bit for bit.  An fp8 cache's
scales get 4x headroom over the generated pool's (the stored codes stay as
they are): a scale set from a small pool's largest value can be exceeded by
the step's freshly drawn new tokens, which E5M2 then stores as infinities
(kernel and oracle alike), and attention over an infinite key is NaN.

PKV_RANDOM_SEEDS=N runs each test on N seeds instead of its default count
(for long sweeps; the draws are the same functions of the seed)."""

import os
from dataclasses import replace

import numpy as np
import pytest

import oracle
from paged_kv_cache_336_amd import workloads as W
from paged_kv_cache_336_amd.step import DeviceStep, MultiStep

from parity_helpers import (TOL, assert_pools_bitwise, check_attention,
                            max_abs_err, oracle_out, oracle_pools, say)

pytestmark = pytest.mark.gpu

_SEEDS = int(os.environ.get("PKV_RANDOM_SEEDS", "0"))


def seeds(default):
    return range(_SEEDS if _SEEDS > 0 else default)

KINDS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
         ("bf16", "fp8_e4m3"), ("f16", "fp8_e5m2"), ("f32", "fp8_e4m3"),
         ("bf16", "fp8_e5m2")]


def _lengths(rng, n, bs, cap):
    lens = rng.integers(1, cap, size=n)
    for i in range(n):
        r = rng.random()
        if r < 0.12:
            lens[i] = 0                        # an empty sequence
        elif r < 0.24:
            lens[i] = bs * int(rng.integers(1, max(2, cap // bs)))  # on a block
        elif r < 0.36:
            lens[i] = 32 * int(rng.integers(1, max(2, cap // 32))) + 1
    return [int(x) for x in lens]


def draw_decode(seed):
    rng = np.random.default_rng([336, 900, seed])
    q, kv = KINDS[int(rng.integers(len(KINDS)))]
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 20]))
    while hkv * g > 64:
        hkv //= 2
    hkv = max(hkv, 1)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([1, 3, 7, 16, 32, 48, 64]))
    n = int(rng.integers(1, 13))
    lens = _lengths(rng, n, bs, 1500)
    waves = int(rng.choice([0, 4, 8, 24, 100]))
    per_head = kv.startswith("fp8") and bool(rng.random() < 0.5)
    return dict(q=q, kv=kv, hq=hkv * g, hkv=hkv, d=d, bs=bs, lens=lens,
                waves=waves, per_head=per_head)


def draw_multi(seed):
    rng = np.random.default_rng([336, 901, seed])
    q, kv = KINDS[int(rng.integers(len(KINDS)))]
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([3, 16, 32, 48]))
    n = int(rng.integers(1, 7))
    lens = [max(1, L) for L in _lengths(rng, n, bs, 900)]
    qlens = []
    for L in lens:
        r = rng.random()
        qlens.append(L if r < 0.15 else (0 if r < 0.25 else
                                          int(rng.integers(1, min(L, 260) + 1))))
    waves = int(rng.choice([0, 8, 40]))
    per_head = kv.startswith("fp8") and bool(rng.random() < 0.5)
    return dict(q=q, kv=kv, hq=hkv * g, hkv=hkv, d=d, bs=bs, lens=lens,
                qlens=qlens, waves=waves, per_head=per_head)


@pytest.mark.parametrize("seed", seeds(32))
def test_random_decode(seed):
    c = draw_decode(seed)
    say(f"random decode {seed}: {c}")
    w = W.custom_decode(seed=1000 + seed, num_seqs=len(c["lens"]),
                        lens=c["lens"], hq=c["hq"], hkv=c["hkv"], d=c["d"],
                        bs=c["bs"], q_kind=c["q"], kv_kind=c["kv"],
                        per_head_scales=c["per_head"])
    if c["kv"].startswith("fp8"):
        w = replace(w, k_scale=np.float32(4) * w.k_scale,
                    v_scale=np.float32(4) * w.v_scale)
    dev = DeviceStep(w, replicas=False)
    dev.copy()
    dev.write()
    pools = oracle_pools(w)
    assert_pools_bitwise(dev, pools)  # the step's copies and writes
    err, out = check_attention(dev, w, pools, max_waves=c["waves"])
    say(f"  max abs err {err:.3g}")
    # rows of empty sequences are zeros
    for s, L in enumerate(c["lens"]):
        if L == 0:
            assert not out[s].any()


@pytest.mark.parametrize("seed", seeds(16))
def test_random_multi(seed):
    import torch
    c = draw_multi(seed)
    say(f"random multi {seed}: {c}")
    mq = W.custom_multi(seed=2000 + seed, lens=c["lens"], qlens=c["qlens"],
                        hq=c["hq"], hkv=c["hkv"], d=c["d"], bs=c["bs"],
                        q_kind=c["q"], kv_kind=c["kv"],
                        per_head_scales=c["per_head"])
    if c["kv"].startswith("fp8"):
        mq = replace(mq, w=replace(mq.w, k_scale=np.float32(4) * mq.w.k_scale,
                                   v_scale=np.float32(4) * mq.w.v_scale))
    dev = MultiStep(mq)
    dev.copy()
    dev.write()
    dev.attend(max_waves=c["waves"])
    torch.cuda.synchronize()
    w = mq.w
    kp, vp = oracle_pools(w)
    assert_pools_bitwise(dev, (kp, vp))  # the step's copies and writes
    ref = oracle.paged_attention_multi(
        mq.query, w.q_kind, kp, vp, w.kv_kind, w.block_tables, w.seq_lens,
        mq.query_start, w.block_size, w.scale, w.k_scale, w.v_scale)
    assert np.isfinite(ref).all(), "the inputs overflow the cache type"
    err = max_abs_err(dev.out.cpu().numpy(), ref)
    say(f"  max abs err {err:.3g}")
    assert err <= TOL[c["kv"]], f"{err:.3g}"


@pytest.mark.parametrize("seed", seeds(12))
def test_random_fused_equals_separate(seed):
    """The fused write + attention on random shapes (G up to 16, uniform and
    other block sizes) against the separate write and decode: the same
    output and pools bit for bit; the separate pair against the oracle
    (pools bit for bit, output within tolerance)."""
    from test_gpu_fused import assert_same, run_pair
    c = draw_decode(100 + seed)
    while c["hq"] // c["hkv"] > 16:
        c["hq"] //= 2
        c["hq"] = max(c["hq"], c["hkv"]) // c["hkv"] * c["hkv"]
    say(f"random fused {seed}: {c}")
    w = W.custom_decode(seed=3000 + seed, num_seqs=len(c["lens"]),
                        lens=c["lens"], hq=c["hq"], hkv=c["hkv"], d=c["d"],
                        bs=c["bs"], q_kind=c["q"], kv_kind=c["kv"],
                        per_head_scales=c["per_head"])
    if c["kv"].startswith("fp8"):
        w = replace(w, k_scale=np.float32(4) * w.k_scale,
                    v_scale=np.float32(4) * w.v_scale)
    sep, fus = run_pair(w, max_waves=c["waves"])
    assert_same(sep, fus)
    pools = oracle_pools(w)
    assert_pools_bitwise(sep, pools)
    err = max_abs_err(sep.out.cpu().numpy(), oracle_out(w, pools))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL[c["kv"]], f"{err:.3g}"


@pytest.mark.parametrize("seed", seeds(8))
def test_random_token_scales(seed):
    """Per-token fp8 scales on random shapes: the token-scaled write (codes
    and scales bit for bit), then decode, against the oracle's token-scaled
    write and attention."""
    import torch
    from test_gpu_token_scales import assert_scales_bitwise
    c = draw_decode(200 + seed)
    kv = "fp8_e4m3" if seed % 2 == 0 else "fp8_e5m2"
    q = ("bf16", "f16", "f32")[seed % 3]
    say(f"random token scales {seed}: {q}/{kv} {c}")
    w = W.custom_decode(seed=4000 + seed, num_seqs=len(c["lens"]),
                        lens=c["lens"], hq=c["hq"], hkv=c["hkv"], d=c["d"],
                        bs=c["bs"], q_kind=q, kv_kind=kv,
                        per_token_scales=True)
    dev = DeviceStep(w, replicas=False)
    dev.copy()
    dev.write()
    dev.attend(max_waves=c["waves"])
    torch.cuda.synchronize()
    kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
    ks, vs = oracle.copy_token_scales(w.k_scale, w.v_scale, w.copy_pairs)
    kp, vp, ks, vs = oracle.cache_write_token_scales(
        kp, vp, ks, vs, w.kv_kind, w.key, w.value, w.src_kind,
        w.slot_mapping, w.block_size)
    assert_pools_bitwise(dev, (kp, vp))  # codes and each row's scale
    assert_scales_bitwise(dev, ks, vs)
    ref = oracle.paged_attention(w.query, q, kp, vp, kv, w.block_tables,
                                 w.seq_lens, w.block_size, w.scale, ks, vs)
    assert np.isfinite(ref).all()
    err = max_abs_err(dev.out.cpu().numpy(), ref)
    say(f"  max abs err {err:.3g}")
    assert err <= TOL[kv], f"{err:.3g}"


@pytest.mark.parametrize("seed", seeds(16))
def test_random_copies(seed):
    """Whole-block and token-prefix copies (one layer, or several layers in
    one launch) and the per-token scale arrays' copies on random pool
    geometry, random bits in every cache type, random disjoint pairs
    (possibly none) and prefix counts on and past the block's ends: every
    pool and scale array bit for bit against the oracle's copies."""
    import torch
    from paged_kv_cache_336_amd import ops
    from paged_kv_cache_336_amd.step import _to_torch, to_host_storage
    rng = np.random.default_rng([336, 902, seed])
    kind = ["f32", "f16", "bf16", "fp8_e4m3", "fp8_e5m2"][int(rng.integers(5))]
    nl = int(rng.choice([1, 1, 2, 3]))
    nb = int(rng.integers(2, 80))
    bs = int(rng.choice([1, 3, 7, 16, 32, 48, 64]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    say(f"random copies {seed}: {kind} layers {nl} blocks {nb} bs {bs} "
        f"hkv {hkv} d {d}")
    shape = (nl, nb, bs, hkv, d)
    if kind == "f32":
        kp = rng.standard_normal(shape).astype(np.float32)
        vp = rng.standard_normal(shape).astype(np.float32)
    else:
        bits = np.uint8 if kind.startswith("fp8") else np.uint16
        kp = rng.integers(0, np.iinfo(bits).max + 1, shape).astype(bits)
        vp = rng.integers(0, np.iinfo(bits).max + 1, shape).astype(bits)
        if kind == "f16":
            kp, vp = kp.view(np.float16), vp.view(np.float16)
    ks = rng.standard_normal((nb, bs, hkv)).astype(np.float32)
    vs = rng.standard_normal((nb, bs, hkv)).astype(np.float32)

    def disjoint(count):
        """count (src, dst) pairs, no destination also a source"""
        perm = rng.permutation(nb)
        return perm[:count], perm[count:2 * count]

    src, dst = disjoint(int(rng.integers(0, nb // 2 + 1)))
    pairs = np.stack([src, dst], axis=1).astype(np.int32).reshape(-1, 2)
    src, dst = disjoint(int(rng.integers(0, nb // 2 + 1)))
    toks = rng.integers(-2, bs + 3, size=len(src))
    triples = np.stack([src, dst, toks], axis=1).astype(np.int32).reshape(-1, 3)

    kc, vc = _to_torch(kp, kind, "cuda"), _to_torch(vp, kind, "cuda")
    ck = kind if kind.startswith("fp8") else None
    pt, tt = torch.from_numpy(pairs).cuda(), torch.from_numpy(triples).cuda()
    if nl == 1:
        ops.copy_blocks(kc[0], vc[0], pt, cache_kind=ck)
        ops.copy_block_prefixes(kc[0], vc[0], tt, cache_kind=ck)
    else:
        ops.copy_blocks_layers(kc, vc, pt, cache_kind=ck)
        ops.copy_block_prefixes_layers(kc, vc, tt, cache_kind=ck)
    kst, vst = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    ops.copy_token_scales(kst, vst, pt)
    ops.copy_token_scale_prefixes(kst, vst, tt)
    torch.cuda.synchronize()

    gk, gv = to_host_storage(kc, kind), to_host_storage(vc, kind)
    for layer in range(nl):
        ek, ev = oracle.copy_blocks(kp[layer], vp[layer], pairs)
        ek, ev = oracle.copy_block_prefixes(ek, ev, triples)
        assert gk[layer].tobytes() == ek.tobytes(), f"k_cache, layer {layer}"
        assert gv[layer].tobytes() == ev.tobytes(), f"v_cache, layer {layer}"
    eks, evs = oracle.copy_token_scales(ks, vs, pairs)
    eks, evs = oracle.copy_token_scales(eks, evs, triples, prefix=True)
    assert kst.cpu().numpy().tobytes() == eks.tobytes(), "k scales"
    assert vst.cpu().numpy().tobytes() == evs.tobytes(), "v scales"


WRITE_PAIRS = [("f32", "f32"), ("bf16", "bf16"), ("f16", "f16"),
               ("fp8_e4m3", "bf16"), ("fp8_e4m3", "f16"), ("fp8_e4m3", "f32"),
               ("fp8_e5m2", "bf16"), ("fp8_e5m2", "f16"), ("fp8_e5m2", "f32")]


@pytest.mark.parametrize("seed", seeds(16))
def test_random_writes(seed):
    """cache_write_slots on random pool geometry, every supported (cache,
    source) type pairing, per-tensor or per-head fp8 scales over a wide
    range, rows spread over sixty binades with zeros, infinities and NaNs
    among them (fp8 caches), distinct slots with some skipped (-1): both
    pools bit for bit against the oracle's write."""
    import torch
    from paged_kv_cache_336_amd import ops
    from paged_kv_cache_336_amd.step import _to_torch, to_host_storage
    from paged_kv_cache_336_amd.workloads import _cast_from_f32
    rng = np.random.default_rng([336, 903, seed])
    kind, src = WRITE_PAIRS[int(rng.integers(len(WRITE_PAIRS)))]
    fp8 = kind.startswith("fp8")
    nb = int(rng.integers(2, 64))
    bs = int(rng.choice([1, 3, 7, 16, 32, 48, 64]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    n = int(rng.integers(0, nb * bs // 2 + 2))
    per_head = fp8 and bool(rng.random() < 0.5)
    say(f"random writes {seed}: {src} -> {kind} blocks {nb} bs {bs} hkv {hkv} "
        f"d {d} tokens {n} per-head {per_head}")
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    slots[rng.random(n) < 0.15] = -1

    def rows():
        x = rng.standard_normal((n, hkv, d)).astype(np.float64)
        x *= np.exp2(rng.uniform(-30, 30, (n, hkv, 1)))
        if fp8:
            special = rng.random((n, hkv, d)) < 0.03
            x[special] = rng.choice([0.0, -0.0, np.inf, -np.inf, np.nan],
                                    special.sum())
        with np.errstate(over="ignore"):  # (f16 sources: past 65504 is inf)
            return _cast_from_f32(x.astype(np.float32), src)

    key, value = rows(), rows()
    shape = (nb, bs, hkv, d)
    if kind == "f32":
        kp = rng.standard_normal(shape).astype(np.float32)
        vp = rng.standard_normal(shape).astype(np.float32)
    else:
        bits = np.uint8 if fp8 else np.uint16
        kp = rng.integers(0, np.iinfo(bits).max + 1, shape).astype(bits)
        vp = rng.integers(0, np.iinfo(bits).max + 1, shape).astype(bits)
        if kind == "f16":
            kp, vp = kp.view(np.float16), vp.view(np.float16)
    count = hkv if per_head else 1
    k_scale = np.exp2(rng.uniform(-10, 6, count)).astype(np.float32)
    v_scale = np.exp2(rng.uniform(-10, 6, count)).astype(np.float32)

    kc, vc = _to_torch(kp, kind, "cuda"), _to_torch(vp, kind, "cuda")
    kw = {}
    if fp8:
        kw = dict(k_scale=torch.from_numpy(k_scale).cuda(),
                  v_scale=torch.from_numpy(v_scale).cuda(), cache_kind=kind)
    ops.cache_write_slots(_to_torch(key, src, "cuda"),
                          _to_torch(value, src, "cuda"), kc, vc,
                          torch.from_numpy(slots).cuda(), **kw)
    torch.cuda.synchronize()
    sk = (k_scale if per_head else k_scale[0]) if fp8 else 1.0
    sv = (v_scale if per_head else v_scale[0]) if fp8 else 1.0
    ek, ev = oracle.cache_write(kp, vp, kind, key, value, src, slots, bs,
                                sk, sv)
    assert to_host_storage(kc, kind).tobytes() == ek.tobytes(), "k_cache"
    assert to_host_storage(vc, kind).tobytes() == ev.tobytes(), "v_cache"


@pytest.mark.parametrize("seed", seeds(16))
def test_random_token_writes(seed):
    """cache_write_slots_token_scaled on random pool geometry, both fp8
    formats, every source type, rows over sixty binades with zeros,
    infinities and NaNs among them, whole zero rows, distinct slots with
    some skipped: codes and each row's scale bit for bit against the
    oracle's token-scaled write."""
    import torch
    from paged_kv_cache_336_amd import ops
    from paged_kv_cache_336_amd.step import _to_torch, to_host_storage
    from paged_kv_cache_336_amd.workloads import _cast_from_f32
    rng = np.random.default_rng([336, 904, seed])
    kind = ("fp8_e4m3", "fp8_e5m2")[int(rng.integers(2))]
    src = ("f32", "f16", "bf16")[int(rng.integers(3))]
    nb = int(rng.integers(2, 40))
    bs = int(rng.choice([1, 3, 7, 16, 32, 64]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    n = int(rng.integers(0, min(nb * bs // 2 + 2, 160)))
    say(f"random token writes {seed}: {src} -> {kind} blocks {nb} bs {bs} "
        f"hkv {hkv} d {d} tokens {n}")
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    slots[rng.random(n) < 0.15] = -1

    def rows():
        x = rng.standard_normal((n, hkv, d)).astype(np.float64)
        x *= np.exp2(rng.uniform(-30, 30, (n, hkv, 1)))
        special = rng.random((n, hkv, d)) < 0.02
        x[special] = rng.choice([0.0, -0.0, np.inf, -np.inf, np.nan],
                                special.sum())
        x[rng.random((n, hkv)) < 0.05] = 0.0  # whole zero rows
        with np.errstate(over="ignore"):  # (f16 sources: past 65504 is inf)
            return _cast_from_f32(x.astype(np.float32), src)

    key, value = rows(), rows()
    shape = (nb, bs, hkv, d)
    kp = rng.integers(0, 256, shape).astype(np.uint8)
    vp = rng.integers(0, 256, shape).astype(np.uint8)
    ks = rng.standard_normal((nb, bs, hkv)).astype(np.float32)
    vs = rng.standard_normal((nb, bs, hkv)).astype(np.float32)
    kc, vc = _to_torch(kp, kind, "cuda"), _to_torch(vp, kind, "cuda")
    kst, vst = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    ops.cache_write_slots_token_scaled(
        _to_torch(key, src, "cuda"), _to_torch(value, src, "cuda"), kc, vc,
        kst, vst, torch.from_numpy(slots).cuda(), cache_kind=kind)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):  # (an infinity over its row's scale)
        ek, ev, eks, evs = oracle.cache_write_token_scales(
            kp, vp, ks, vs, kind, key, value, src, slots, bs)
    assert to_host_storage(kc, kind).tobytes() == ek.tobytes(), "k codes"
    assert to_host_storage(vc, kind).tobytes() == ev.tobytes(), "v codes"
    assert kst.cpu().numpy().tobytes() == eks.tobytes(), "k scales"
    assert vst.cpu().numpy().tobytes() == evs.tobytes(), "v scales"


@pytest.mark.parametrize("seed", seeds(8))
def test_random_multi_token_scales(seed):
    """Several new tokens per sequence over per-token-scaled fp8 caches on
    random shapes: the token-scaled write (codes and scales bit for bit),
    then the multi-query call, against the oracle."""
    import torch
    from test_gpu_token_scales import assert_scales_bitwise
    c = draw_multi(300 + seed)
    kv = "fp8_e4m3" if seed % 2 == 0 else "fp8_e5m2"
    q = ("bf16", "f16", "f32")[seed % 3]
    say(f"random multi token scales {seed}: {q}/{kv} {c}")
    mq = W.custom_multi(seed=2500 + seed, lens=c["lens"], qlens=c["qlens"],
                        hq=c["hq"], hkv=c["hkv"], d=c["d"], bs=c["bs"],
                        q_kind=q, kv_kind=kv, per_token_scales=True)
    dev = MultiStep(mq, replicas=False)
    dev.copy()
    dev.write()
    dev.attend(max_waves=c["waves"])
    torch.cuda.synchronize()
    w = mq.w
    kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
    ks, vs = oracle.copy_token_scales(w.k_scale, w.v_scale, w.copy_pairs)
    kp, vp, ks, vs = oracle.cache_write_token_scales(
        kp, vp, ks, vs, w.kv_kind, w.key, w.value, w.src_kind,
        w.slot_mapping, w.block_size)
    assert_pools_bitwise(dev, (kp, vp))
    assert_scales_bitwise(dev, ks, vs)
    ref = oracle.paged_attention_multi(
        mq.query, q, kp, vp, kv, w.block_tables, w.seq_lens, mq.query_start,
        w.block_size, w.scale, ks, vs)
    assert np.isfinite(ref).all()
    err = max_abs_err(dev.out.cpu().numpy(), ref)
    say(f"  max abs err {err:.3g}")
    assert err <= TOL[kv], f"{err:.3g}"
