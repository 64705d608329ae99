"""The control half and the hot path together (GPU): a decode loop whose slot
mappings, copy-on-write pairs and block tables come from the C++ block
manager drives copy_blocks -> cache_write_slots -> paged_attn_decode on the
GPU, while the oracle's block manager and operations replay the same steps
on the CPU.  The two managers must agree exactly, the pools bit for bit, and
the attention within the path's tolerance -- through prompts, forks (parallel
sampling), copy-on-write, frees and re-use of freed blocks."""

import numpy as np
import pytest

import oracle
from oracle.block_manager import BlockManager as OracleBM
from paged_kv_cache_336_amd import blocks, ops
from paged_kv_cache_336_amd import workloads as W
from paged_kv_cache_336_amd.step import _to_torch, to_host_storage

from parity_helpers import TOL, max_abs_err, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_kind", ["bf16", "fp8_e4m3"])
def test_decode_loop_driven_by_block_manager(kv_kind):
    import torch
    rng = np.random.default_rng([336, 99, 1 if kv_kind == "bf16" else 2])
    nb, bs, hkv, hq, d = 96, 16, 2, 8, 64
    max_seqs, mbps = 8, 16
    q_kind, src_kind = "bf16", "bf16"
    scale = float(np.float32(1.0 / np.sqrt(d)))
    k_scale = v_scale = 0.5 if kv_kind == "fp8_e4m3" else 1.0
    cache_kind = kv_kind if kv_kind == "fp8_e4m3" else None
    say(f"decode loop: kv={kv_kind} nb={nb} bs={bs} hkv={hkv} hq={hq} d={d}")

    pk = np.full((nb, bs, hkv, d), W.poison_value(kv_kind))
    pv = pk.copy()
    kc, vc = _to_torch(pk, kv_kind, "cuda"), _to_torch(pv, kv_kind, "cuda")
    ks = torch.tensor([k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([v_scale], dtype=torch.float32, device="cuda")
    bm = blocks.BlockManager(nb, bs, max_seqs, mbps)
    ob = OracleBM(nb, bs, mbps)

    def write(slots):
        nonlocal pk, pv
        n = len(slots)
        key = W._cast_from_f32(rng.standard_normal((n, hkv, d), np.float32),
                               src_kind)
        val = W._cast_from_f32(rng.standard_normal((n, hkv, d), np.float32),
                               src_kind)
        sl = np.asarray(slots, dtype=np.int32)
        ops.cache_write_slots(_to_torch(key, src_kind, "cuda"),
                              _to_torch(val, src_kind, "cuda"), kc, vc,
                              torch.from_numpy(sl).cuda(), k_scale=ks,
                              v_scale=vs, cache_kind=cache_kind)
        pk, pv = oracle.cache_write(pk, pv, kv_kind, key, val, src_kind, sl,
                                    bs, k_scale, v_scale)

    prefix = kv_kind == "fp8_e4m3"  # one run copies whole blocks, one only
                                    # the tokens a block holds

    def copy(pairs, counts):
        nonlocal pk, pv
        p = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
        if prefix:
            t = np.concatenate([p, np.asarray(counts, np.int32).reshape(-1, 1)],
                               axis=1)
            ops.copy_block_prefixes(kc, vc, torch.from_numpy(t).cuda(),
                                    cache_kind=cache_kind)
            pk, pv = oracle.copy_block_prefixes(pk, pv, t)
        else:
            ops.copy_blocks(kc, vc, torch.from_numpy(p).cuda(),
                            cache_kind=cache_kind)
            pk, pv = oracle.copy_blocks(pk, pv, p)

    def add(seq, n):
        slots = bm.add_sequence(seq, n)
        assert list(slots) == ob.add_sequence(seq, n)
        write(slots)

    def check_pools():
        torch.cuda.synchronize()
        assert to_host_storage(kc, kv_kind).tobytes() == pk.tobytes()
        assert to_host_storage(vc, kv_kind).tobytes() == pv.tobytes()

    for seq, n in [(0, 37), (1, 5), (2, 100)]:
        add(seq, n)
    for child in (3, 4):            # two more samples of prompt 0
        bm.fork(0, child)
        ob.fork(0, child)
    live = [0, 1, 2, 3, 4]
    out = torch.empty((max_seqs, hq, d), dtype=torch.float32, device="cuda")
    copies = 0
    for step in range(40):
        if step == 15:
            bm.free(1)
            ob.free_sequence(1)
            live.remove(1)
        if step == 20:
            add(5, 20)              # takes blocks freed by sequence 1
            live.append(5)
        slots, pairs, counts = bm.append(live, with_counts=True)
        want_slots, want_pairs, want_counts = ob.append(live, True)
        assert list(slots) == want_slots
        assert [tuple(p) for p in pairs] == want_pairs
        assert list(counts) == want_counts
        copies += len(pairs)
        copy(pairs, counts)         # copy-on-write before the new token
        write(slots)
        tab, lens = bm.tables(live, fill=0)
        q = W._cast_from_f32(rng.standard_normal((len(live), hq, d),
                                                 np.float32), q_kind)
        o = out[:len(live)]
        ops.paged_attn_decode(o, _to_torch(q, q_kind, "cuda"), kc, vc,
                              torch.from_numpy(tab).cuda(),
                              torch.from_numpy(lens).cuda(), int(lens.max()),
                              scale, k_scale=ks, v_scale=vs,
                              cache_kind=cache_kind)
        torch.cuda.synchronize()
        ref = oracle.paged_attention(q, q_kind, pk, pv, kv_kind, tab, lens, bs,
                                     scale, k_scale, v_scale)
        err = max_abs_err(o.cpu().numpy(), ref)
        assert err <= TOL[kv_kind], f"step {step}: {err:.3g}"
        if step % 10 == 9:
            check_pools()
    check_pools()
    assert copies == 2              # 0 and 3 copied; 4, the last sharer, kept it
    assert bm.stats() == ob.stats()
    say(f"decode loop: {kv_kind} ok, {copies} copy-on-write pairs")


def test_prefix_cached_prompts_share_blocks_and_results():
    """Two requests with the same system prompt: the second one's leading
    full blocks come from the prefix cache, so only its remaining prompt
    tokens are written and attended as new queries (paged_attn_multi).  Its
    output equals, bit for bit, the same request run on private blocks with
    every prompt token written, and the oracle within tolerance."""
    import torch
    nb, bs, hkv, hq, d = 48, 16, 2, 8, 128
    kind = "bf16"
    scale = float(np.float32(1.0 / np.sqrt(d)))

    def kv_row(prefix):
        # a K/V row fixed by the tokens up to and including its position
        # (as a model's would be), so equal prefixes give equal rows
        r = np.random.default_rng([336, 7] + [int(t) for t in prefix])
        return r.standard_normal((2, hkv, d), np.float32)

    rng = np.random.default_rng(123)
    system = [int(t) for t in rng.integers(0, 1000, 40)]     # 2.5 blocks
    prompt_a = system + [int(t) for t in rng.integers(0, 1000, 10)]
    prompt_b = system + [int(t) for t in rng.integers(0, 1000, 7)]
    kc = _to_torch(np.full((nb, bs, hkv, d), W.poison_value(kind)), kind, "cuda")
    vc = kc.clone()
    bm = blocks.BlockManager(nb, bs, 4, 8, prefix_cache=True)

    def prefill(seq, prompt):
        slots, cached = bm.add_sequence_tokens(seq, prompt)
        n = len(prompt)
        rows = np.stack([kv_row(prompt[:p + 1]) for p in range(cached, n)])
        key = W._cast_from_f32(rows[:, 0], kind)
        val = W._cast_from_f32(rows[:, 1], kind)
        ops.cache_write_slots(_to_torch(key, kind, "cuda"),
                              _to_torch(val, kind, "cuda"), kc, vc,
                              torch.from_numpy(slots[cached:].copy()).cuda())
        q = W._cast_from_f32(rng.standard_normal((n - cached, hq, d),
                                                 np.float32), kind)
        tab, lens = bm.tables([seq], fill=0)
        out = torch.empty((n - cached, hq, d), dtype=torch.float32,
                          device="cuda")
        qs = torch.tensor([0, n - cached], dtype=torch.int32, device="cuda")
        ops.paged_attn_multi(out, _to_torch(q, kind, "cuda"), kc, vc,
                             torch.from_numpy(tab).cuda(),
                             torch.from_numpy(lens).cuda(), qs, n - cached,
                             n, scale)
        torch.cuda.synchronize()
        return cached, q, tab, lens, out.cpu().numpy()

    say("prefix cache: request A (no cache), request B (system prompt cached)")
    ca, _, tab_a, _, _ = prefill(0, prompt_a)
    cb, qb, tab_b, lens_b, out_b = prefill(1, prompt_b)
    assert ca == 0 and cb == 32
    assert list(tab_b[0, :2]) == list(tab_a[0, :2])        # shared blocks
    assert bm.refcount(int(tab_a[0, 0])) == 2
    # the oracle on the shared pools
    pk = to_host_storage(kc, kind)
    pv = to_host_storage(vc, kind)
    ref = oracle.paged_attention_multi(qb, kind, pk, pv, kind, tab_b, lens_b,
                                       np.array([0, len(qb)]), bs, scale)
    assert max_abs_err(out_b, ref) <= TOL[kind]
    # the same request on private blocks, every prompt token written
    priv = blocks.BlockManager(nb, bs, 4, 8)
    slots_p = priv.add_sequence(1, len(prompt_b))
    n = len(prompt_b)
    rows = np.stack([kv_row(prompt_b[:p + 1]) for p in range(n)])
    kc2 = _to_torch(np.full((nb, bs, hkv, d), W.poison_value(kind)), kind,
                    "cuda")
    vc2 = kc2.clone()
    ops.cache_write_slots(_to_torch(W._cast_from_f32(rows[:, 0], kind), kind,
                                    "cuda"),
                          _to_torch(W._cast_from_f32(rows[:, 1], kind), kind,
                                    "cuda"), kc2, vc2,
                          torch.from_numpy(slots_p).cuda())
    tab_p, lens_p = priv.tables([1], fill=0)
    out2 = torch.empty((n - 32, hq, d), dtype=torch.float32, device="cuda")
    ops.paged_attn_multi(out2, _to_torch(qb, kind, "cuda"), kc2, vc2,
                         torch.from_numpy(tab_p).cuda(),
                         torch.from_numpy(lens_p).cuda(),
                         torch.tensor([0, n - 32], dtype=torch.int32,
                                      device="cuda"), n - 32, n, scale)
    torch.cuda.synchronize()
    assert np.array_equal(out2.cpu().numpy().view(np.uint32),
                          out_b.view(np.uint32))
    say(f"prefix cache: {bm.prefix_stats()}")
