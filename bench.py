"""Benchmark of the paged KV-cache decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: copy_blocks (the
copy-on-write pairs of the batch; none for a plain decode batch), then the
new token of every sequence written into its slot and paged decode attention
-- in one launch (paged_attn_decode_fused) where the batch allows it, else
cache_write_slots followed by paged_attn_decode.
Inputs are seeded synthetic tensors already resident in HBM; steps rotate
over disjoint replicas of the block tables where the workload has them, so
the 256 MB Infinity Cache cannot serve one step's K/V to the next.

Timing is GPU time: before each timed region the GPU is kept busy by a
calibrated spin kernel while the host enqueues the region's work, so the
region's events bracket back-to-back kernels and not host launch gaps.

Prints one JSON line: KV-read GB/s of the whole step (value), tokens/s, the
attention call's roofline fraction against 8 TB/s and the CPU oracle's rate
on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1, "fp8_e5m2": 1}
DTYPE_NAME = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8",
              "fp8_e5m2": "fp8_e5m2"}
METRIC = ("paged decode attention KV-read GB/s (% of HBM peak) + "
          "decode tokens/s, 1 GPU")


def algorithmic_bytes(w):
    """Bytes each call must move.  Attention reads every live K and V row
    of every sequence once (logical bytes: a block shared by several
    sequences counts once per sequence), the query, the block-table entries
    and lengths, and writes the float32 output."""
    e = ELEM_BYTES[w.kv_kind]
    eq = ELEM_BYTES[w.q_kind]
    L = w.seq_lens.astype(np.int64)
    hkv, d, bs = w.num_kv_heads, w.head_dim, w.block_size
    S, hq = w.num_seqs, w.num_q_heads
    attn = int(L.sum()) * hkv * d * e * 2 + S * hq * d * (eq + 4) + \
        int(((L + bs - 1) // bs).sum()) * 4 + 4 * S
    es = ELEM_BYTES[w.src_kind]
    T = w.num_tokens
    write = T * hkv * d * (es + e) * 2 + 4 * T
    if np.ndim(w.k_scale) == 3:   # fp8 scales per token: 4 B per row read
        attn += int(L.sum()) * hkv * 4 * 2                   # and written
        write += T * hkv * 4 * 2
    copy = 2 * len(w.copy_pairs) * bs * hkv * d * e * 2
    return {"attention": attn, "cache_write": write, "copy_blocks": copy}


DECODE_SOURCES = ("attn_decode.hip", "attn_tile.h", "pkv_device.h",
                  "pkv_internal.h")
MULTI_SOURCES = ("attn_multi.hip", "attn_tile.h", "pkv_device.h",
                 "pkv_internal.h")


def kernel_source_sha(sources=DECODE_SOURCES):
    """Hash of the sources the attention kernels are built from: a traffic
    record taken with other sources no longer describes the kernel."""
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "paged_kv_cache_336_amd", "csrc", name),
                  "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def seq_bytes(w, s):
    """Algorithmic attention bytes of sequence s alone."""
    e, eq = ELEM_BYTES[w.kv_kind], ELEM_BYTES[w.q_kind]
    L = int(w.seq_lens[s])
    return (L * w.num_kv_heads * w.head_dim * e * 2 +
            w.num_q_heads * w.head_dim * (eq + 4) +
            -(-L // w.block_size) * 4 + 4)


def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on replica 0 of the same workload.

    When a whole step (copy, write, attention over the batch) fits the
    budget, whole steps are repeated until it is used and the rate is the
    step's.  Otherwise the sample is attention over sequences 0, 1, 2, ...
    (all their heads, on the pools after the step's copy and write), one at a
    time until the budget is used, and the rate is those sequences' bytes
    over their attention time.  Returns (value GB/s, tokens/s, sample text,
    threads)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()]
                      or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))

    # fp8 scales per (slot, kv head) travel with the pools: the copy and the
    # token-scaled write update them, and attention reads the updated ones
    token_scales = np.ndim(w.k_scale) == 3
    scales = {}

    def prepare():
        kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
        if token_scales:
            ks, vs = oracle.copy_token_scales(w.k_scale, w.v_scale,
                                              w.copy_pairs)
            kp, vp, scales["k"], scales["v"] = oracle.cache_write_token_scales(
                kp, vp, ks, vs, w.kv_kind, w.key, w.value, w.src_kind,
                w.slot_mapping, w.block_size)
            return kp, vp
        scales["k"], scales["v"] = w.k_scale, w.v_scale
        return oracle.cache_write(kp, vp, w.kv_kind, w.key, w.value,
                                  w.src_kind, w.slot_mapping, w.block_size,
                                  w.k_scale, w.v_scale)

    def attend(kp, vp, lo, hi):
        oracle.paged_attention(w.query[lo:hi], w.q_kind, kp, vp, w.kv_kind,
                               w.block_tables[lo:hi], w.seq_lens[lo:hi],
                               w.block_size, w.scale, scales["k"], scales["v"])

    t0 = time.perf_counter()
    kp, vp = prepare()
    t_prep = time.perf_counter() - t0
    t0 = time.perf_counter()
    attend(kp, vp, 0, 1)
    t_one = time.perf_counter() - t0
    # attention time scales with the tokens attended
    est = t_prep + t_one * float(w.seq_lens.sum()) / max(int(w.seq_lens[0]), 1)
    B = algorithmic_bytes(w)["attention"]
    if est < budget_s / 2:
        steps = 0
        t0 = time.perf_counter()
        while True:
            kp, vp = prepare()
            attend(kp, vp, 0, w.num_seqs)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        return (B * steps / el / 1e9, w.num_seqs * steps / el,
                f"{steps} whole step(s) of {w.name} (replica 0, "
                f"{w.num_seqs} sequences, the full batch) in {el:.1f} s",
                threads)
    nbytes, n, el = seq_bytes(w, 0), 1, t_one
    while el < budget_s and n < w.num_seqs:
        t0 = time.perf_counter()
        attend(kp, vp, n, n + 1)
        el += time.perf_counter() - t0
        nbytes += seq_bytes(w, n)
        n += 1
    return (nbytes / el / 1e9, n / el,
            f"attention of sequences 0..{n - 1} of {w.name} (replica 0, all "
            f"{w.num_q_heads} query heads, {nbytes / 1e6:.1f} MB of the "
            f"batch's {B / 1e6:.1f} MB) in {el:.1f} s; copy and write of the "
            f"step ran once beforehand, untimed", threads)


def multi_algorithmic(mq):
    """Bytes and flops one paged_attn_multi call must move / do: every live
    K and V row of every sequence read once, the new tokens' queries read
    and their float32 outputs written, the tables, lengths and query starts;
    flops 2 * 2 * D per (query head, visible key) -- Q.K and P.V -- over the
    causal extent of each new token."""
    w = mq.w
    e, eq = ELEM_BYTES[w.kv_kind], ELEM_BYTES[w.q_kind]
    L = w.seq_lens.astype(np.int64)
    q = np.diff(mq.query_start).astype(np.int64)
    hkv, d, bs, hq = w.num_kv_heads, w.head_dim, w.block_size, w.num_q_heads
    T = int(q.sum())
    nbytes = (int(L.sum()) * hkv * d * e * 2 + T * hq * d * (eq + 4) +
              int(((L + bs - 1) // bs).sum()) * 4 + 4 * (2 * len(L) + 1))
    # token j of q new ones sees L - q + j + 1 keys: sum = q (L - q) + q (q+1)/2
    visible = int((q * (L - q) + q * (q + 1) // 2).sum())
    flops = 4 * d * hq * visible
    write = T * hkv * d * (ELEM_BYTES[w.src_kind] + e) * 2 + 4 * T
    return {"attention": nbytes, "flops": flops, "cache_write": write}


def multi_seq_cost(mq, s):
    """(bytes, new tokens) of sequence s alone."""
    w = mq.w
    e, eq = ELEM_BYTES[w.kv_kind], ELEM_BYTES[w.q_kind]
    L = int(w.seq_lens[s])
    q = int(mq.query_start[s + 1] - mq.query_start[s])
    return (L * w.num_kv_heads * w.head_dim * e * 2 +
            q * w.num_q_heads * w.head_dim * (eq + 4) +
            -(-L // w.block_size) * 4 + 12, q)


def cpu_baseline_multi(mq, budget_s):
    """The oracle on replica 0: attention of sequences 0, 1, 2, ... (all new
    tokens, all heads, on the pools after the step's write) one at a time,
    going round the batch again if it ends first, until the budget is used.
    Returns (GB/s, new tokens/s, sample text, threads)."""
    import oracle
    w = mq.w
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()]
                      or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    kp, vp = oracle.cache_write(w.k_pool, w.v_pool, w.kv_kind, w.key,
                                w.value, w.src_kind, w.slot_mapping,
                                w.block_size, w.k_scale, w.v_scale)
    qs = mq.query_start
    nbytes = ntok = n = 0
    el = 0.0
    while el < budget_s or n == 0:
        i = n % w.num_seqs
        t0 = time.perf_counter()
        oracle.paged_attention_multi(
            mq.query[qs[i]:qs[i + 1]], w.q_kind, kp, vp, w.kv_kind,
            w.block_tables[i:i + 1], w.seq_lens[i:i + 1],
            np.asarray([0, qs[i + 1] - qs[i]]), w.block_size, w.scale,
            w.k_scale, w.v_scale)
        el += time.perf_counter() - t0
        b, q = multi_seq_cost(mq, i)
        nbytes += b
        ntok += q
        n += 1
    what = (f"sequences 0..{n - 1}" if n <= w.num_seqs else
            f"{n} sequences ({n / w.num_seqs:.2f} passes over the batch)")
    return (nbytes / el / 1e9, ntok / el,
            f"attention of {what} of {w.name} (replica 0, {ntok} new "
            f"tokens, all {w.num_q_heads} query heads, "
            f"{nbytes / 1e6:.1f} MB) in {el:.1f} s; the step's write ran "
            f"once beforehand, untimed", threads)


def contiguous_table_sets(w, count):
    """Block tables that give every sequence consecutive physical blocks
    (sequence after sequence), in up to `count` disjoint ranges of the pool:
    the unpaged layout the paging overhead is measured against.  Only the
    addresses matter for that measurement, not what the blocks hold.  Empty
    when the pool cannot hold every sequence's blocks unshared (a batch whose
    sequences share blocks can need more than the pool has)."""
    L = w.seq_lens.astype(np.int64)
    bs = w.block_size
    nblk = (L + bs - 1) // bs
    need = int(nblk.sum())
    count = min(count, w.num_blocks // max(need, 1))
    first = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    sets = []
    for r in range(count):
        t = np.zeros_like(w.block_tables)
        for s in range(w.num_seqs):
            t[s, :nblk[s]] = r * need + first[s] + np.arange(nblk[s])
        if int(t.min()) < 0 or int(t.max()) >= w.num_blocks:
            raise AssertionError("contiguous table entry outside the pool")
        sets.append(t)
    return sets


class GpuClock:
    """Keeps the GPU busy with torch's spin kernel while the host enqueues a
    timed region, so that region runs back to back on the GPU."""

    def __init__(self, torch):
        self.torch = torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        n = 2_000_000
        torch.cuda._sleep(n)          # warm
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        self.cycles_per_ms = n / max(a.elapsed_time(b), 1e-3)

    def hold(self, ms):
        self.torch.cuda._sleep(int(self.cycles_per_ms * ms))


def timed_region(torch, clock, enqueue, host_ms_estimate):
    """GPU milliseconds of the work enqueue() issues, measured with events
    recorded after a spin long enough to cover the host's enqueueing."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clock.hold(2.0 * host_ms_estimate + 5.0)
    start.record()
    h0 = time.perf_counter()
    enqueue()
    host_ms = (time.perf_counter() - h0) * 1e3
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop), host_ms


def copy_calibration(nbytes):
    """Three plain device-to-device copies of nbytes each: under rocprofv3
    --pmc their FETCH_SIZE / WRITE_SIZE readings against the known byte count
    give the factor that turns those counters into bytes."""
    import torch
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes,
                                           "bytes_written": nbytes,
                                           "copies": 3}}), flush=True)


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
MULTI_METRIC = ("paged multi-query attention (causal new tokens) KV-read GB/s "
                "+ TFLOP/s, 1 GPU")


def warm_and_estimate(torch, step, warmup):
    """Warm-up steps; returns the host's enqueue time per step (ms)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(max(warmup, 1)):
        step(i)
    ms = (time.perf_counter() - h0) * 1e3 / max(warmup, 1)
    torch.cuda.synchronize()
    return ms


def load_traffic(path, workload, sources):
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if rec and rec.get("kernel_source_sha") == kernel_source_sha(sources):
        return rec.get("bytes_per_call")
    return None


def bench_multi(args):
    """Steps of several new tokens per sequence: cache_write_slots of the
    new tokens, then paged_attn_multi."""
    import torch
    from paged_kv_cache_336_amd import workloads as W
    from paged_kv_cache_336_amd.step import MultiStep

    mq = W.MULTI_WORKLOADS[args.workload](replicas=args.replicas)
    w = mq.w
    # the library's choice of partition kernel: workgroup rows of 16
    # column groups for 12 or more groups of new tokens on a 16-bit cache
    # the queries share, block_size % 16 == 0
    G = w.num_q_heads // w.num_kv_heads
    long_rows = (w.q_kind == w.kv_kind and w.kv_kind in ("bf16", "f16") and
                 w.block_size % 16 == 0 and
                 -(-mq.max_query_len // (16 // G)) >= 12)
    dev = MultiStep(mq, device="cuda:0")
    R = len(dev.sets)
    cost = multi_algorithmic(mq)
    K = args.steps

    def step(i):
        dev.write(i % R)
        dev.attend(i % R, max_waves=args.max_waves)

    host_step_ms = warm_and_estimate(torch, step, args.warmup)
    clock = GpuClock(torch)
    step_total, host_ms = timed_region(
        torch, clock, lambda: [step(i) for i in range(K)], host_step_ms * K)
    ms_step = step_total / K
    attn_total, _ = timed_region(
        torch, clock,
        lambda: [dev.attend(i % R, max_waves=args.max_waves)
                 for i in range(K)], host_step_ms * K)
    attn_ms = attn_total / K
    write_total, _ = timed_region(
        torch, clock, lambda: [dev.write(i % R) for i in range(K)],
        host_step_ms * K)
    write_ms = write_total / K

    B, F = cost["attention"], cost["flops"]
    T = int(mq.query.shape[0])
    peak_tf = MFMA_PEAK_TFLOPS[w.q_kind]
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBPS * 1e9)   # flop per byte
    attn_gbps = B / (attn_ms * 1e-3) / 1e9
    attn_tflops = F / (attn_ms * 1e-3) / 1e12
    if F / B > ridge:
        roof = {"bound": "mfma", "achieved": round(attn_tflops, 2),
                "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(attn_tflops / peak_tf, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(attn_gbps, 2),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(attn_gbps / HBM_PEAK_GBPS, 4)}
    roof.update({
        "kernel": "paged_attn_multi (" + (
            "attn_prefill_kernel" if long_rows else "attn_multi_kernel") +
            " + attn_multi_merge_kernel)",
        "traffic": load_traffic(args.traffic_json, args.workload,
                                MULTI_SOURCES),
        "algorithmic_bytes_per_launch": B,
        "algorithmic_flops_per_launch": F,
        "kv_read_gbps": round(attn_gbps, 2),
        "tflops": round(attn_tflops, 3),
        "flop_per_byte": round(F / B, 2),
        "ridge_flop_per_byte": round(ridge, 1),
    })
    cpu = None
    if not args.no_cpu_baseline:
        gbps, tps, sample, threads = cpu_baseline_multi(mq, args.cpu_budget)
        cpu = {"value": round(gbps, 4), "unit": "GB/s",
               "cores": int(threads), "kind": "oracle", "sample": sample,
               "new_tokens_per_s": round(tps, 2)}
    line = {
        "metric": MULTI_METRIC,
        "value": round(B / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.kv_kind],
        "data": "synthetic (seeded N(0,1) values)",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs,
            "new_tokens": T,
            "max_query_len": mq.max_query_len,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "kv_dtype": w.kv_kind,
            "q_dtype": w.q_kind,
            "sum_seq_len": int(w.seq_lens.sum()),
            "max_seq_len": w.max_seq_len,
            "replicas": R,
            "max_waves": args.max_waves,
        },
        "new_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "tflops_step": round(F / (ms_step * 1e-3) / 1e12, 3),
        "attention_us": round(attn_ms * 1e3, 3),
        "cache_write_us": round(write_ms * 1e3, 3),
        "cache_write_gbps": round(cost["cache_write"] / (write_ms * 1e-3)
                                  / 1e9, 2),
        "host_enqueue_ms": round(host_ms, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def workload_kwargs(name, replicas):
    """Generator arguments: the 8B-shaped batch is small (101 MB of K/V), so
    it rotates over disjoint replicas that together exceed the 256 MB
    Infinity Cache; the larger batches (1.7 GB, 2.1 GB) need none."""
    return {"replicas": replicas} if name == "llama8b_decode" else {}


def attention_only(args, name):
    """The attention call of another decode workload: K calls back to back
    between one event pair, rotating over its replicas, with its algorithmic
    bytes and roofline fraction (reported beside the main line)."""
    import torch
    from paged_kv_cache_336_amd import workloads as W
    from paged_kv_cache_336_amd.step import DeviceStep
    w = W.workload_by_name(name, **workload_kwargs(name, args.replicas))
    dev = DeviceStep(w, device="cuda:0")
    R = len(dev.sets)
    K = args.steps

    def run_attn():
        for i in range(K):
            dev.attend(i % R, max_waves=args.max_waves)
    host_ms = warm_and_estimate(torch, lambda i: dev.attend(
        i % R, max_waves=args.max_waves), args.warmup)
    clock = GpuClock(torch)
    total, enqueue_ms = timed_region(torch, clock, run_attn, host_ms * K)
    ms = total / K
    B = algorithmic_bytes(w)["attention"]
    gbps = B / (ms * 1e-3) / 1e9
    rec = {"workload": w.name, "attention_us": round(ms * 1e3, 3),
           "algorithmic_bytes_per_launch": B, "achieved_gbps": round(gbps, 2),
           "frac": round(gbps / HBM_PEAK_GBPS, 4),
           "host_us_per_attention_call": round(enqueue_ms * 1e3 / K, 2),
           "kv_stream_hint": bool(dev.sets[0]["kv_stream"]),
           "replicas": R}
    del dev, w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama70b_decode",
                    help="llama70b_decode (default: the largest single-GPU "
                    "decode batch at 16-bit precision), llama8b_decode, "
                    "prefix_sharing_{fork,divergent}_bs{32,544}, "
                    "long_context_fp8, worked_example; several new tokens "
                    "per sequence: spec_verify_llama8b, "
                    "chunked_prefill_llama8b")
    ap.add_argument("--also", default="llama8b_decode,long_context_fp8",
                    help="comma-separated decode workloads whose attention "
                    "call is also timed and reported beside the main line "
                    "(\"\" for none)")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--max-waves", type=int, default=0,
                    help="cap on the attention kernel's waves (0 = all)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--token-scales", action="store_true",
                    help="long_context_fp8 with fp8 scales per (slot, kv "
                    "head) instead of per tensor")
    ap.add_argument("--unfused", action="store_true",
                    help="time the step as separate write and attention "
                    "calls even where they can go in one launch")
    ap.add_argument("--no-paging-overhead", action="store_true",
                    help="skip the contiguous-table comparison")
    ap.add_argument("--traffic-json", default=os.path.join(
        ROOT, "profiles", "traffic.json"))
    ap.add_argument("--copy-calibration", type=int, default=0,
                    metavar="BYTES", help="only run plain copies of BYTES "
                    "(byte-counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the hot path runs on one GPU (asked for "
              f"{args.gpus}); splitting it across GPUs is described, not "
              "measured", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    from paged_kv_cache_336_amd import ops
    from paged_kv_cache_336_amd import workloads as W
    from paged_kv_cache_336_amd.step import DeviceStep

    ops.load_library()
    if args.workload in W.MULTI_WORKLOADS:
        bench_multi(args)
        return
    kw = workload_kwargs(args.workload, args.replicas)
    if args.token_scales:
        if args.workload != "long_context_fp8":
            sys.exit("bench.py: --token-scales applies to long_context_fp8")
        kw["per_token_scales"] = True
    w = W.workload_by_name(args.workload, **kw)
    token_scales = np.ndim(w.k_scale) == 3
    dev = DeviceStep(w, device="cuda:0")
    R = len(dev.sets)
    nbytes = algorithmic_bytes(w)
    K = args.steps

    # the write and the attention go in one launch where the batch has one
    # new token per (non-empty) sequence and at most 16 query heads per kv
    # head; else as two calls
    fused = (not args.unfused and not token_scales and
             w.num_tokens == w.num_seqs and
             bool((w.seq_lens > 0).all()) and
             w.num_q_heads // w.num_kv_heads <= 16)

    def step(i):
        r = i % R
        dev.copy(r)
        if fused:
            dev.attend_fused(r, max_waves=args.max_waves)
        else:
            dev.write(r)
            dev.attend(r, max_waves=args.max_waves)

    def step_unfused(i):
        r = i % R
        dev.copy(r)
        dev.write(r)
        dev.attend(r, max_waves=args.max_waves)

    # warm-up; also estimates the host's enqueue time per step
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(max(args.warmup, 1)):
        step(i)
    host_step_ms = (time.perf_counter() - h0) * 1e3 / max(args.warmup, 1)
    torch.cuda.synchronize()
    clock = GpuClock(torch)

    # ---- timed region: K whole steps, rotating replicas ----
    def run_steps():
        for i in range(K):
            step(i)
    step_ms_total, host_ms = timed_region(torch, clock, run_steps,
                                          host_step_ms * K)
    ms_step = step_ms_total / K
    unfused_ms = ms_step
    if fused:
        for i in range(max(args.warmup, 1)):
            step_unfused(i)
        unfused_total, _ = timed_region(
            torch, clock, lambda: [step_unfused(i) for i in range(K)],
            host_step_ms * K)
        unfused_ms = unfused_total / K

    # ---- the same steps through prepared calls: arguments marshalled once,
    # as a serving loop whose tensors stay in place issues them ----
    dev.prepare(fused=fused, max_waves=args.max_waves)
    for i in range(max(args.warmup, 1)):
        dev.step_prepared(i % R)
    torch.cuda.synchronize()
    prep_total, prep_host_ms = timed_region(
        torch, clock, lambda: [dev.step_prepared(i % R) for i in range(K)],
        host_step_ms * K)
    prep_ms = prep_total / K

    # ---- the attention call alone: K calls back to back between one event
    # pair on the stream the kernels run on (torch's current stream) ----
    def run_attn():
        for i in range(K):
            dev.attend(i % R, max_waves=args.max_waves)
    attn_total, attn_host_ms = timed_region(torch, clock, run_attn,
                                           host_step_ms * K)
    attn_avg_ms = attn_total / K
    attn_calls = [dev.attend(r, max_waves=args.max_waves, prepare=True)
                  for r in range(R)]
    _, attn_prep_host_ms = timed_region(
        torch, clock, lambda: [attn_calls[i % R]() for i in range(K)],
        host_step_ms * K)

    # ---- paging overhead: the same calls with contiguous block tables ----
    paging = None
    csets = [] if args.no_paging_overhead else [
        torch.from_numpy(t).to("cuda:0") for t in contiguous_table_sets(w, R)]
    if not args.no_paging_overhead and not csets:
        paging = {"skipped": "the pool cannot hold every sequence's blocks "
                             "unshared"}
    if csets:

        def run_contig():
            for i in range(K):
                ops.paged_attn_decode(dev.out, dev.query, dev.k_cache,
                                      dev.v_cache, csets[i % len(csets)],
                                      dev.seq_lens, dev.max_seq_len, w.scale,
                                      k_scale=dev.k_scale, v_scale=dev.v_scale,
                                      max_waves=args.max_waves,
                                      workspace=dev.workspace,
                                      cache_kind=dev.cache_kind,
                                      kv_stream=dev.sets[0]["kv_stream"])
        run_contig()
        contig_total, _ = timed_region(torch, clock, run_contig,
                                       host_step_ms * K)
        contig_ms = contig_total / K
        paging = {"contiguous_tables_us": round(contig_ms * 1e3, 3),
                  "paged_tables_us": round(attn_avg_ms * 1e3, 3),
                  "gbps_ratio_contiguous_over_paged":
                      round(attn_avg_ms / contig_ms, 4),
                  "contiguous_table_sets": len(csets)}

    # ---- the cache write alone (for the report) ----
    def run_write():
        for i in range(K):
            dev.write(i % R)
    write_total, _ = timed_region(torch, clock, run_write, host_step_ms * K)
    write_ms = write_total / K

    # ---- the copy-on-write copies alone (when the batch has any) ----
    copy_ms = 0.0
    if len(w.copy_pairs):
        def run_copy():
            for i in range(K):
                dev.copy(i % R)
        copy_total, _ = timed_region(torch, clock, run_copy, host_step_ms * K)
        copy_ms = copy_total / K

    B = nbytes["attention"]
    step_gbps = B / (ms_step * 1e-3) / 1e9
    attn_gbps = B / (attn_avg_ms * 1e-3) / 1e9
    tokens_per_s = w.num_seqs / (ms_step * 1e-3)

    traffic = load_traffic(args.traffic_json, args.workload +
                           ("_token_scales" if token_scales else ""),
                           DECODE_SOURCES)

    cpu = None
    if not args.no_cpu_baseline:
        gbps, tps, sample, threads = cpu_baseline(w, args.cpu_budget)
        cpu = {"value": round(gbps, 4), "unit": "GB/s",
               "cores": int(threads), "kind": "oracle", "sample": sample,
               "tokens_per_s": round(tps, 2)}

    line = {
        "metric": METRIC,
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.kv_kind],
        "data": "synthetic (seeded N(0,1) values, lognormal lengths)",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "kv_dtype": w.kv_kind,
            "q_dtype": w.q_kind,
            "kv_scales": ("per token" if token_scales else
                          "per kv head" if np.size(w.k_scale) > 1 else
                          "per tensor") if w.kv_kind.startswith("fp8")
                         else None,
            "sum_seq_len": int(w.seq_lens.sum()),
            "max_seq_len": w.max_seq_len,
            "replicas": R,
            "max_waves": args.max_waves,
            # PKV_KV_STREAM: passed when no block is read by two sequences
            "kv_stream_hint": bool(dev.sets[0]["kv_stream"]),
        },
        "step": ("copy_blocks + paged_attn_decode_fused (write and "
                 "attention in one launch)" if fused else
                 "copy_blocks + cache_write_slots + paged_attn_decode"),
        "step_us_separate_write": round(unfused_ms * 1e3, 3),
        "tokens_per_s": round(tokens_per_s, 1),
        "hbm_frac_step": round(step_gbps / HBM_PEAK_GBPS, 4),
        "attention_us": round(attn_avg_ms * 1e3, 3),
        "cache_write_us": round(write_ms * 1e3, 3),
        "cache_write_gbps": round(nbytes["cache_write"] / (write_ms * 1e-3)
                                  / 1e9, 2),
        "copy_blocks_us": round(copy_ms * 1e3, 3),
        "copy_blocks_gbps": (round(nbytes["copy_blocks"] / (copy_ms * 1e-3)
                                   / 1e9, 2) if copy_ms > 0 else None),
        "host_enqueue_ms": round(host_ms, 3),
        "host_us_per_step": round(host_ms * 1e3 / K, 2),
        "host_us_per_attention_call": round(attn_host_ms * 1e3 / K, 2),
        "prepared": {"ms_per_step": round(prep_ms, 5),
                     "host_us_per_step": round(prep_host_ms * 1e3 / K, 2),
                     "host_us_per_attention_call":
                         round(attn_prep_host_ms * 1e3 / K, 2),
                     "note": "the same calls with their arguments "
                             "marshalled once (ops prepare=True)"},
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_attn_decode (attn_decode_kernel + attn_merge_kernel)",
            "achieved": round(attn_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": B,
        },
        "cpu_baseline": cpu,
        "paging_overhead": paging,
    }
    others = [n for n in args.also.split(",") if n and n != args.workload
              and n in W.DECODE_WORKLOADS] if not args.token_scales else []
    if others:
        del dev
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        line["other_workloads"] = [attention_only(args, n) for n in others]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
