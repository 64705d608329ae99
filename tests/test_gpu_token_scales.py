"""Per-token fp8 scales through the C ABI on the GPU: the token-scaled write
(codes and each row's scale) and the scale-array copies bit for bit against
the oracle; decode and multi-query attention over per-token-scaled pools
within the fp8 tolerance, for both fp8 formats, all query types, uniform
and non-uniform block sizes, several wave splits, rows of zeros and NaN
elements, and scales spread over forty binades."""

import numpy as np
import pytest

import oracle
from paged_kv_cache_336_amd import ops
from paged_kv_cache_336_amd import workloads as W
from paged_kv_cache_336_amd.step import DeviceStep, MultiStep, _to_torch

from parity_helpers import TOL, assert_pools_bitwise, max_abs_err, say

pytestmark = pytest.mark.gpu


def oracle_state(w):
    """Pools and scale arrays after this step's copies and writes."""
    kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
    ks, vs = oracle.copy_token_scales(w.k_scale, w.v_scale, w.copy_pairs)
    return oracle.cache_write_token_scales(kp, vp, ks, vs, w.kv_kind, w.key,
                                           w.value, w.src_kind,
                                           w.slot_mapping, w.block_size)


def assert_scales_bitwise(dev, ks, vs):
    got_k = dev.k_scale.cpu().numpy()
    got_v = dev.v_scale.cpu().numpy()
    assert got_k.view(np.uint32).tobytes() == ks.view(np.uint32).tobytes()
    assert got_v.view(np.uint32).tobytes() == vs.view(np.uint32).tobytes()


def step(w, max_waves=0, multi=None):
    import torch
    dev = MultiStep(multi, replicas=False) if multi is not None else \
        DeviceStep(w, replicas=False)
    assert dev.token_scales
    dev.copy()
    dev.write()
    dev.attend(max_waves=max_waves)
    torch.cuda.synchronize()
    return dev


CASES = [
    # (q, kv, d, bs, hq, hkv, lens, waves)
    ("bf16", "fp8_e4m3", 128, 16, 32, 8, [1, 15, 16, 17, 300, 2500], 0),
    ("bf16", "fp8_e4m3", 128, 64, 16, 4, [63, 64, 65, 4000], 8),
    ("f16", "fp8_e5m2", 128, 16, 8, 8, [33, 700], 4),
    ("f32", "fp8_e4m3", 64, 32, 4, 2, [1, 90, 640], 0),
    ("f32", "fp8_e5m2", 64, 16, 2, 1, [31, 32, 129], 4),
    ("bf16", "fp8_e5m2", 64, 7, 12, 2, [9, 64, 130], 0),    # bs % 16 != 0
    ("f16", "fp8_e4m3", 128, 5, 16, 16, [3, 77], 4),
    ("bf16", "fp8_e4m3", 128, 16, 64, 4, [40, 1000], 0),    # 16 heads per kv
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"{c[0]}-{c[1]}-D{c[2]}-bs{c[3]}-G{c[4] // c[5]}-L{max(c[6])}-W{c[7]}"
    for c in CASES])
def test_token_scaled_decode(case):
    q, kv, d, bs, hq, hkv, lens, waves = case
    say(f"token-scaled decode {case}")
    w = W.custom_decode(seed=900 + CASES.index(case), num_seqs=len(lens),
                        lens=lens, hq=hq, hkv=hkv, d=d, bs=bs, q_kind=q,
                        kv_kind=kv, per_token_scales=True)
    assert np.asarray(w.k_scale).shape == w.k_pool.shape[:3]
    kp, vp, ks, vs = oracle_state(w)
    for wv in sorted({0, waves}):
        dev = step(w, max_waves=wv)
        assert_pools_bitwise(dev, (kp, vp))
        assert_scales_bitwise(dev, ks, vs)
        ref = oracle.paged_attention(w.query, q, kp, vp, kv, w.block_tables,
                                     w.seq_lens, bs, w.scale, ks, vs)
        err = max_abs_err(dev.out.cpu().numpy(), ref)
        say(f"  waves {wv}: max abs err {err:.3g}")
        assert err <= TOL[kv], f"waves {wv}: {err:.3g}"


@pytest.mark.parametrize("kv", ["fp8_e4m3", "fp8_e5m2"])
@pytest.mark.parametrize("src", ["f32", "f16", "bf16"])
def test_token_scaled_write_edge_rows(kv, src):
    """Rows of zeros, rows with NaN elements, magnitudes over many binades
    and skipped slots: codes and scales bit for bit."""
    import torch
    say(f"token-scaled write {src} -> {kv}")
    rng = np.random.default_rng(31)
    nb, bs, hkv, d, T = 9, 16, 4, 128, 40
    x = rng.standard_normal((2, T, hkv, d)).astype(np.float32)
    x *= np.exp2(rng.uniform(-14, 14, (2, T, hkv, 1))).astype(np.float32)
    x[:, 3] = 0.0                                   # all-zero rows
    x[0, 5, 1, 17] = np.nan                         # a NaN among values
    x[1, 6, 2, :] = 0.0
    x[1, 6, 2, 40] = np.nan                         # NaN among zeros
    x[0, 7, 0, 9] = -1e4                            # one large element
    key = W._cast_from_f32(x[0], src)
    value = W._cast_from_f32(x[1], src)
    slots = rng.permutation(nb * bs)[:T].astype(np.int32)
    slots[[2, 11]] = -1                             # skipped
    kp0 = np.full((nb, bs, hkv, d), 0x7F, dtype=np.uint8)
    ks0 = np.full((nb, bs, hkv), np.nan, dtype=np.float32)
    kp, vp, ks, vs = oracle.cache_write_token_scales(
        kp0, kp0.copy(), ks0, ks0.copy(), kv, key, value, src, slots, bs)
    dk = _to_torch(kp0, kv, "cuda")
    dv = _to_torch(kp0.copy(), kv, "cuda")
    dks = torch.from_numpy(ks0.copy()).cuda()
    dvs = torch.from_numpy(ks0.copy()).cuda()
    ops.cache_write_slots_token_scaled(
        _to_torch(key, src, "cuda"), _to_torch(value, src, "cuda"), dk, dv,
        dks, dvs, torch.from_numpy(slots).cuda(), cache_kind=kv)
    torch.cuda.synchronize()
    assert dk.cpu().numpy().tobytes() == kp.tobytes()
    assert dv.cpu().numpy().tobytes() == vp.tobytes()
    assert dks.cpu().numpy().view(np.uint32).tobytes() == \
        ks.view(np.uint32).tobytes()
    assert dvs.cpu().numpy().view(np.uint32).tobytes() == \
        vs.view(np.uint32).tobytes()


@pytest.mark.parametrize("kv", ["fp8_e4m3", "fp8_e5m2"])
def test_token_scales_over_forty_binades(kv):
    """Value scales multiplied by 2^k, k in [-20, 20], and key scales by
    2^k, k in [-3, 3] (exact in float32), row by row: the PV weights are
    formed against the running maximum of score + log2(value scale), so
    the result stays within the fp8 tolerance relative to each output row's
    size."""
    import torch
    say(f"token scales over forty binades {kv}")
    w = W.custom_decode(seed=950, num_seqs=4, lens=[7, 200, 1300, 64],
                        hq=16, hkv=4, d=128, bs=16, q_kind="bf16",
                        kv_kind=kv, per_token_scales=True)
    kp, vp, ks, vs = oracle_state(w)
    rng = np.random.default_rng(951)
    ks = ks * np.exp2(rng.integers(-3, 4, ks.shape)).astype(np.float32)
    vs = vs * np.exp2(rng.integers(-20, 21, vs.shape)).astype(np.float32)
    dev = DeviceStep(w, replicas=False)
    dev.k_cache.copy_(_to_torch(kp, kv, "cuda"))
    dev.v_cache.copy_(_to_torch(vp, kv, "cuda"))
    dev.k_scale.copy_(torch.from_numpy(ks))
    dev.v_scale.copy_(torch.from_numpy(vs))
    for wv in (0, 8):
        dev.attend(max_waves=wv)
        torch.cuda.synchronize()
        out = dev.out.cpu().numpy().astype(np.float64)
        ref = oracle.paged_attention(w.query, "bf16", kp, vp, kv,
                                     w.block_tables, w.seq_lens, 16, w.scale,
                                     ks, vs)
        assert np.isfinite(out).all()
        size = np.maximum(1.0, np.abs(ref).max(axis=-1, keepdims=True))
        rel = float(np.max(np.abs(out - ref) / size))
        say(f"  waves {wv}: max error / row size {rel:.3g}")
        assert rel <= TOL[kv], f"waves {wv}: {rel:.3g}"


@pytest.mark.parametrize("kv", ["fp8_e4m3", "fp8_e5m2"])
def test_token_scaled_multi(kv):
    say(f"token-scaled multi-query {kv}")
    mq = W.custom_multi(seed=960, lens=[300, 1200, 9, 64, 517],
                        qlens=[3, 100, 9, 1, 40], hq=8, hkv=2, d=128, bs=16,
                        q_kind="bf16", kv_kind=kv, per_token_scales=True)
    w = mq.w
    kp, vp, ks, vs = oracle_state(w)
    ref = oracle.paged_attention_multi(mq.query, "bf16", kp, vp, kv,
                                       w.block_tables, w.seq_lens,
                                       mq.query_start, w.block_size, w.scale,
                                       ks, vs)
    for wv in (0, 12):
        dev = step(w, max_waves=wv, multi=mq)
        assert_scales_bitwise(dev, ks, vs)
        err = max_abs_err(dev.out.cpu().numpy(), ref)
        say(f"  waves {wv}: max abs err {err:.3g}")
        assert err <= TOL[kv], f"waves {wv}: {err:.3g}"


def test_token_scaled_multi_f32_queries_any_block_size():
    mq = W.custom_multi(seed=961, lens=[50, 333, 8], qlens=[11, 29, 8],
                        hq=6, hkv=2, d=64, bs=7, q_kind="f32",
                        kv_kind="fp8_e4m3", per_token_scales=True)
    w = mq.w
    kp, vp, ks, vs = oracle_state(w)
    dev = step(w, multi=mq)
    ref = oracle.paged_attention_multi(mq.query, "f32", kp, vp, "fp8_e4m3",
                                       w.block_tables, w.seq_lens,
                                       mq.query_start, w.block_size, w.scale,
                                       ks, vs)
    assert max_abs_err(dev.out.cpu().numpy(), ref) <= TOL["fp8_e4m3"]


@pytest.mark.parametrize("prefix", [False, True])
def test_scale_copies_bitwise(prefix):
    import torch
    rng = np.random.default_rng(970)
    nb, bs, hkv = 40, 7, 3                     # blocks of 84 bytes
    ks = rng.standard_normal((nb, bs, hkv)).astype(np.float32)
    vs = rng.standard_normal((nb, bs, hkv)).astype(np.float32)
    perm = rng.permutation(nb)
    src, dst = perm[:12], perm[12:24]
    if prefix:
        recs = np.stack([src, dst, rng.integers(-2, 10, 12)], 1)
    else:
        recs = np.stack([src, dst], 1)
    recs = recs.astype(np.int32)
    eks, evs = oracle.copy_token_scales(ks, vs, recs, prefix=prefix)
    dks, dvs = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    fn = ops.copy_token_scale_prefixes if prefix else ops.copy_token_scales
    fn(dks, dvs, torch.from_numpy(recs).cuda())
    torch.cuda.synchronize()
    assert dks.cpu().numpy().tobytes() == eks.tobytes()
    assert dvs.cpu().numpy().tobytes() == evs.tobytes()


def test_long_context_token_scaled_full():
    """A long-context batch (4 x 32768 tokens, bs 64, bf16 queries,
    per-token E4M3 scales) in the default launch configuration; every
    (sequence, query head) row against the oracle."""
    say("token-scaled long context")
    w = W.long_context_fp8(num_seqs=4, seq_len=32768, per_token_scales=True)
    kp, vp, ks, vs = oracle_state(w)
    dev = step(w)
    rows = [(s, h) for s in range(4) for h in range(32)]
    ref = oracle.paged_attention_rows(w.query, "bf16", kp, vp, "fp8_e4m3",
                                      w.block_tables, w.seq_lens, 64,
                                      w.scale, rows, ks, vs)
    out = dev.out.cpu().numpy()
    got = np.stack([out[s, h] for s, h in rows])
    err = max_abs_err(got, ref)
    say(f"  max abs err {err:.3g}")
    assert err <= TOL["fp8_e4m3"]
