"""KV-memory waste: contiguous max-length reservation against paging.

    python -m paged_kv_cache_336_amd.waste [--seqs N] [--median M] [--cap C]

Drives the two host allocators of libpagedkv.so (include/pagedkv_blocks.h)
over synthetic lengths and prints the three comparisons "PagedAttention"
(shubhamtatvamasi.com) makes:

* introduction: a request reserving its maximum length (8K) that answers in
  300 tokens leaves more than 96% of its reservation unused;
* "Choosing the block size" and its figure: over long-tailed lengths, the
  contiguous waste depends on how far the maximum length sits above typical
  lengths, the paged waste only on the block size (at most one partial block
  per sequence), and smaller blocks mean more block-table entries;
* "The idea: page the KV cache" and its animation: five requests over 64
  token slots; reserving 20 slots each admits three and makes two wait,
  while blocks handed out one at a time admit all five.

The page prints no numbers for the figure or the animation; the lengths here
are the seeded lognormal draws of the decode workloads (sigma 1) and a fixed
set of five short answers, so the output reproduces the shape of the claims,
not the page's pixels.
"""

import argparse

import numpy as np

from .blocks import BlockManager, ContiguousAllocator
from . import workloads as W


def reservation_waste(answer_tokens, max_len):
    """Fraction of one max_len reservation left unused by an answer."""
    ca = ContiguousAllocator(max_len, 1)
    assert ca.reserve(0, max_len) == 0
    return 1.0 - answer_tokens / ca.stats()["reserved_slots"]


def contiguous_waste(lengths, max_len):
    """Unused fraction of one max_len reservation per sequence (max_len
    must hold the longest sequence)."""
    assert int(np.max(lengths)) <= max_len
    n = len(lengths)
    ca = ContiguousAllocator(n * max_len, n)
    for i in range(n):
        assert ca.reserve(i, max_len) is not None
    reserved = ca.stats()["reserved_slots"]
    return 1.0 - float(np.sum(lengths)) / reserved


def paged_waste(lengths, block_size):
    """(unused fraction of the allocated block slots, mean block-table
    entries per sequence) with each sequence's blocks taken on demand."""
    lengths = [int(x) for x in lengths]
    need = sum(-(-L // block_size) for L in lengths)
    longest = max(-(-L // block_size) for L in lengths)
    bm = BlockManager(max(need, 1), block_size, len(lengths), max(longest, 1))
    for i, L in enumerate(lengths):
        bm.add_sequence(i, L)
    st = bm.stats()
    waste = st["wasted_slots"] / (st["used_blocks"] * block_size)
    return waste, need / len(lengths)


def block_size_sweep(lengths, block_sizes, max_lens):
    rows = []
    for bs in block_sizes:
        w, entries = paged_waste(lengths, bs)
        rows.append({"block_size": bs, "paged_waste": w,
                     "table_entries": entries})
    contiguous = {m: contiguous_waste(lengths, m) for m in max_lens}
    return rows, contiguous


def five_requests(final_lengths=(7, 12, 5, 9, 10), slots=64, reserve=20,
                  block_size=4):
    """The page's animation as a simulation.  Contiguous: each request
    reserves `reserve` slots on arrival, in order; one that finds no gap
    waits.  Paged: every request is admitted and grows one token per step,
    taking a block only when its last one is full."""
    names = "ABCDE"[:len(final_lengths)]
    ca = ContiguousAllocator(slots, len(final_lengths))
    cont_admitted = [names[i] for i in range(len(final_lengths))
                     if ca.reserve(i, reserve) is not None]
    bm = BlockManager(slots // block_size, block_size, len(final_lengths),
                      slots // block_size)
    for i in range(len(final_lengths)):
        bm.add_sequence(i, 0)
    for step in range(max(final_lengths)):
        growing = [i for i, L in enumerate(final_lengths) if L > step]
        bm.append(growing)
    tabs, lens = bm.tables(list(range(len(final_lengths))))
    per_request_waste = [int(-(-L // block_size) * block_size - L)
                         for L in lens]
    return {"contiguous_admitted": cont_admitted,
            "contiguous_waiting": [n for n in names
                                   if n not in cont_admitted],
            "paged_admitted": list(names),
            "paged_blocks_used": bm.stats()["used_blocks"],
            "paged_blocks_total": slots // block_size,
            "paged_waste_per_request": per_request_waste,
            "contiguous_reserved_unused": reserve * len(cont_admitted)
            - sum(final_lengths[i] for i in range(len(cont_admitted)))}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--seqs", type=int, default=4096)
    ap.add_argument("--median", type=int, default=512)
    ap.add_argument("--cap", type=int, default=8192)
    ap.add_argument("--seed", type=int, default=336)
    args = ap.parse_args(argv)

    print("reservation: 8192-token maximum, 300-token answer -> "
          f"{100 * reservation_waste(300, 8192):.1f}% of the reservation unused")

    rng = np.random.default_rng([args.seed, 0])
    lengths = W.lognormal_lengths(rng, args.seqs, args.median, args.cap)
    rows, contiguous = block_size_sweep(
        lengths, [1, 2, 4, 8, 16, 32, 64, 128, 256],
        [args.cap, 2 * args.cap, 4 * args.cap])
    print(f"\n{args.seqs} lognormal lengths (median {args.median}, cap "
          f"{args.cap}, mean {np.mean(lengths):.0f})")
    print(f"{'block size':>10} {'paged waste':>12} {'table entries':>14}")
    for r in rows:
        print(f"{r['block_size']:>10} {100 * r['paged_waste']:>11.2f}% "
              f"{r['table_entries']:>14.1f}")
    for m, w in contiguous.items():
        print(f"contiguous reservation of {m} tokens: {100 * w:.1f}% unused")

    f = five_requests()
    print("\nfive requests, 64 slots: contiguous (20 each) admits "
          f"{''.join(f['contiguous_admitted'])}, "
          f"{''.join(f['contiguous_waiting'])} wait; paged (block 4) admits "
          f"all, using {f['paged_blocks_used']} of {f['paged_blocks_total']} "
          f"blocks, waste per request {f['paged_waste_per_request']}")


if __name__ == "__main__":
    main()
