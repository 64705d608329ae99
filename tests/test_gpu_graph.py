"""The decode step recorded as HIP graphs (DeviceStep.capture: copy_blocks,
cache_write_slots and paged_attn_decode, or the fused call, one graph per
replica set) against the same calls made one by one, through the C ABI on
the GPU.  Every replay -- several rounds, with other eager work queued and
synchronised between them -- must give the eager output bit for bit and
leave the pools as the eager steps left them.  Prepared calls (arguments
marshalled once) give the direct calls' bits, also after the workspace they
were made with has been grown by a larger call."""

import numpy as np
import pytest

from paged_kv_cache_336_amd import workloads as W
from paged_kv_cache_336_amd.step import DeviceStep

from parity_helpers import TOL, max_abs_err, oracle_out, oracle_pools, say

pytestmark = pytest.mark.gpu

CASES = [
    ("8B-shaped, 3 replicas, separate write",
     lambda: W.llama8b_decode(num_seqs=12, median=300, cap=1500,
                              num_blocks=4096, replicas=3), False),
    ("8B-shaped, 2 replicas, fused write",
     lambda: W.llama8b_decode(num_seqs=12, median=300, cap=1500,
                              num_blocks=4096, replicas=2), True),
    ("fp8 long context, small",
     lambda: W.long_context_fp8(num_seqs=2, seq_len=6000), False),
    ("prefix sharing fork (copy-on-write copies)",
     lambda: W.prefix_sharing(block_size=32, phase="fork", groups=2,
                              samples=3, prompt_len=500, max_tail=100)[0],
     False),
]


@pytest.mark.parametrize("label,make,fused", CASES,
                         ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager_steps(label, make, fused):
    import torch
    say(f"graph step: {label}")
    w = make()
    dev = DeviceStep(w, device="cuda:0")
    R = len(dev.sets)

    def eager(r):
        dev.copy(r)
        if fused:
            dev.attend_fused(r)
        else:
            dev.write(r)
            dev.attend(r)

    refs = []
    for r in range(R):
        eager(r)
        torch.cuda.synchronize()
        refs.append(dev.out.clone())
    if R == 1 or not fused:
        # the first set's eager output against the oracle (its own tables;
        # the pools then hold every set's writes, which set 0 never reads)
        pools = oracle_pools(w)
        assert max_abs_err(refs[0].cpu().numpy(),
                           oracle_out(w, pools)) <= TOL[w.kv_kind]
    k_ref, v_ref = dev.k_cache.clone(), dev.v_cache.clone()

    dev.capture(fused=fused)
    for rnd in range(3):
        for r in range(R):
            dev.out.fill_(float("nan"))
            torch.cuda.synchronize()
            dev.replay(r)
            torch.cuda.synchronize()
            assert torch.equal(dev.out.view(torch.int32),
                               refs[r].view(torch.int32)), (rnd, r)
            # other eager work between replays
            dev.attend((r + 1) % R)
            torch.cuda.synchronize()
            assert torch.equal(dev.out.view(torch.int32),
                               refs[(r + 1) % R].view(torch.int32))
    assert torch.equal(dev.k_cache.view(torch.uint8), k_ref.view(torch.uint8))
    assert torch.equal(dev.v_cache.view(torch.uint8), v_ref.view(torch.uint8))
    assert np.isfinite(refs[0].cpu().numpy()).all()


@pytest.mark.parametrize("fused", [False, True])
def test_prepared_calls_equal_direct_calls(fused):
    """DeviceStep.prepare's calls (ops.PreparedCall, arguments marshalled
    once) issue exactly the direct calls: same output bits and pools, every
    replica set, several rounds; a prepared call with a bad argument reports
    the same status as the direct call."""
    import torch
    from paged_kv_cache_336_amd import ops
    w = W.llama8b_decode(num_seqs=12, median=300, cap=1500, num_blocks=4096,
                         replicas=2)
    say(f"prepared calls, fused={fused}")
    direct = DeviceStep(w, device="cuda:0")
    prep = DeviceStep(w, device="cuda:0")
    prep.prepare(fused=fused)
    R = len(direct.sets)
    for rnd in range(2):
        for r in range(R):
            direct.copy(r)
            if fused:
                direct.attend_fused(r)
            else:
                direct.write(r)
                direct.attend(r)
            prep.step_prepared(r)
            torch.cuda.synchronize()
            assert torch.equal(direct.out.view(torch.int32),
                               prep.out.view(torch.int32)), (rnd, r)
    assert torch.equal(direct.k_cache.view(torch.uint8),
                       prep.k_cache.view(torch.uint8))
    assert torch.equal(direct.v_cache.view(torch.uint8),
                       prep.v_cache.view(torch.uint8))
    # a negative wave cap is refused the same way (PKV_ERR_SHAPE)
    bad = prep.attend(0, max_waves=-1, prepare=True)
    with pytest.raises(ops.PagedKVError) as e:
        bad()
    assert e.value.status == 2


def test_prepared_call_keeps_its_workspace_after_growth():
    """A prepared call made with a shared Workspace keeps the buffer it was
    marshalled with: a later, larger call grows the Workspace (a new buffer),
    memory allocated afterwards is not the old buffer, and the prepared call
    still gives its first output bit for bit without touching that memory."""
    import torch
    from paged_kv_cache_336_amd import ops
    small = W.custom_decode(seed=81, num_seqs=3, lens=[700, 40, 1300], hq=32,
                            hkv=8, d=128, bs=16, q_kind="bf16", kv_kind="bf16")
    big = W.custom_decode(seed=82, num_seqs=64, lens=[300] * 64, hq=32,
                          hkv=8, d=128, bs=16, q_kind="bf16", kv_kind="bf16")
    say("prepared call across workspace growth")
    d1 = DeviceStep(small, replicas=False)
    d2 = DeviceStep(big, replicas=False)
    ws = ops.Workspace(torch.device("cuda:0"))

    def decode(dev, prepare):
        return ops.paged_attn_decode(
            dev.out, dev.query, dev.k_cache, dev.v_cache,
            dev.sets[0]["block_tables"], dev.seq_lens, dev.max_seq_len,
            dev.w.scale, max_waves=40, workspace=ws, prepare=prepare)

    call = decode(d1, True)
    old = ws.buf
    nbytes = old.numel()
    call()
    torch.cuda.synchronize()
    ref = d1.out.clone()
    decode(d2, False)                       # grows the shared workspace
    torch.cuda.synchronize()
    assert ws.buf is not old and ws.buf.numel() > nbytes
    del old
    guard = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda:0")
    d1.out.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    assert torch.equal(d1.out.view(torch.int32), ref.view(torch.int32))
    assert bool((guard == 0x5A).all())
