/*
 * pagedkv_blocks.h -- host-side block manager for the paged KV pool, and the
 * contiguous max-length reservation it replaces (kept as the baseline that
 * waste comparisons are made against).  Plain C ABI, no GPU calls: the
 * manager decides which physical blocks a sequence owns; the device calls of
 * pagedkv.h (copy_blocks, cache_write_slots, paged_attn_decode) consume its
 * slot mappings, copy pairs and block tables.
 *
 * What the manager does follows "PagedAttention" (shubhamtatvamasi.com):
 *   - section "The idea: page the KV cache": blocks are handed out one at a
 *     time from a free list, a new one only when a sequence's last block is
 *     full, so a sequence wastes at most one partially filled block;
 *   - section "Sharing and copy-on-write" and the FAQ entry on copy-on-write
 *     for parallel sampling: every block has a reference count equal to the
 *     number of sequences whose table holds it; a sequence about to append
 *     into a shared, partially filled last block first takes a new block,
 *     copies the existing tokens into it, drops its reference to the old one
 *     and writes into the copy; full blocks are never written again and stay
 *     shared.
 * The contiguous allocator follows the same page's introduction (a request
 * reserves room for its maximum length up front; free space splits into gaps)
 * and its animation of five requests over 64 token slots.
 *
 * Allocation order (fixed, so that any two runs, and the test oracle, hand
 * out the same physical blocks): the free list is a stack.  It starts with
 * blocks num_blocks-1 .. 0 pushed in that order, so the first allocations
 * return 0, 1, 2, ...; a freed sequence pushes its blocks whose count drops
 * to zero in logical-block order, so they come back last-freed first.
 *
 * Ownership and errors: handles are created and destroyed by the caller;
 * output arrays are caller-owned host memory.  A call that fails returns a
 * non-zero pkv_status (pagedkv.h) and changes nothing.  A handle is not
 * thread-safe: one thread at a time per handle.
 */
#ifndef PAGEDKV_BLOCKS_H
#define PAGEDKV_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* A manager for a pool of num_blocks blocks of block_size tokens, for
 * sequences with ids 0 .. max_seqs-1 of at most max_blocks_per_seq blocks.
 * Returns NULL for a non-positive argument or when memory runs out. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t max_seqs, int32_t max_blocks_per_seq);
void pkv_bm_destroy(pkv_block_manager* bm);

/* A manager as above that also caches prompt prefixes ("PagedAttention",
 * shubhamtatvamasi.com, "Sharing and copy-on-write": different requests with
 * the same system prompt share blocks).  Every full block that
 * pkv_bm_add_sequence_tokens fills from a prompt is registered under the
 * contents of the prompt up to and including it; a later prompt whose leading
 * full blocks have registered contents takes those blocks (one more
 * reference each) instead of new ones, so its K/V for those tokens are
 * already in the pool.  Partially filled blocks are never shared this way.
 * A registered block whose last reference is dropped stays registered, on an
 * evictable list (oldest release first); allocations take plain free blocks
 * first and reuse evictable ones (dropping their registration) only when
 * none is left.  Readings: a prompt's lookup stops at its first block that
 * is not registered; blocks filled by pkv_bm_append (no token ids) are not
 * registered. */
pkv_block_manager* pkv_bm_create_prefix_cached(int32_t num_blocks,
                                               int32_t block_size,
                                               int32_t max_seqs,
                                               int32_t max_blocks_per_seq);

/* Start sequence seq with num_tokens tokens (a prompt, num_tokens >= 0):
 * takes ceil(num_tokens / block_size) blocks.  slots_out (may be NULL) gets
 * the slot block * block_size + offset of each token, for cache_write_slots.
 * PKV_ERR_SEQ if seq is live, PKV_ERR_SHAPE if seq is out of range or the
 * sequence would need more than max_blocks_per_seq blocks, PKV_ERR_NO_BLOCKS
 * if the free list is too short. */
int pkv_bm_add_sequence(pkv_block_manager* bm, int32_t seq, int32_t num_tokens,
                        int32_t* slots_out);

/* Start sequence seq with the prompt tokens[0 .. num_tokens-1] (token ids).
 * As pkv_bm_add_sequence, except that with a prefix-caching manager the
 * leading full blocks whose contents are registered are shared, and
 * *cached_tokens_out (may be NULL) gets the number of leading tokens whose
 * K/V those blocks already hold: the caller writes and computes only the
 * tokens from there on.  slots_out still gets every token's slot.  Without
 * prefix caching this is pkv_bm_add_sequence with *cached_tokens_out = 0.
 * PKV_ERR_NULL if tokens is NULL with num_tokens > 0. */
int pkv_bm_add_sequence_tokens(pkv_block_manager* bm, int32_t seq,
                               const int32_t* tokens, int32_t num_tokens,
                               int32_t* slots_out, int32_t* cached_tokens_out);

/* Prefix-cache counters: blocks registered (in use or evictable), blocks on
 * the evictable list (no reference, still registered; they also count as
 * free in pkv_bm_get_stats), and prompt blocks found in the cache so far.
 * Any pointer may be NULL. */
int pkv_bm_prefix_stats(const pkv_block_manager* bm, int64_t* registered,
                        int64_t* evictable, int64_t* hit_blocks);

/* Sequence child (not live) starts as a copy of sequence parent (live): the
 * same length and table, and every block of it gains a reference.  No block
 * is taken. */
int pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t child);

/* Append one token to each of the n distinct live sequences seqs[0..n-1], in
 * that order.  For each: if it has no block or its last block is full, it
 * takes a new block; else, if its last block is shared, copy-on-write: it
 * takes a new block, the pair {old, new} is recorded, and its reference to
 * old is dropped (so a later sharer in the same batch whose count has fallen
 * to one writes in place).  slot_mapping[i] gets the new token's slot;
 * pairs_out[2k], pairs_out[2k+1] get the k-th {src, dst} pair (capacity n
 * pairs) and *num_pairs_out their count; copy_tokens_out[k] (may be NULL)
 * the number of tokens the copy must carry (those src holds), for
 * copy_block_prefixes.  All or nothing: PKV_ERR_NO_BLOCKS
 * if the batch needs more blocks than are free, PKV_ERR_SEQ for a sequence
 * that is not live or listed twice, PKV_ERR_SHAPE if one would exceed
 * max_blocks_per_seq. */
int pkv_bm_append(pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                  int32_t* slot_mapping, int32_t* pairs_out,
                  int32_t* num_pairs_out, int32_t* copy_tokens_out);

/* End sequence seq: every block of it loses a reference; blocks left with
 * none return to the free list. */
int pkv_bm_free(pkv_block_manager* bm, int32_t seq);

/* Block tables and lengths of the n live sequences seqs[]: row i of tables
 * (row_stride >= max_blocks_per_seq int32 entries) gets the sequence's
 * physical blocks in logical order followed by fill up to row_stride;
 * lens[i] (may be NULL) its token count.  The rows are the block_tables and
 * seq_lens arguments of paged_attn_decode. */
int pkv_bm_tables(const pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                  int32_t* tables, int32_t row_stride, int32_t fill,
                  int32_t* lens);

/* Whether an attention call over the n live sequences seqs[] may carry the
 * PKV_KV_STREAM hint (pagedkv.h): *unshared = 1 when no physical block
 * appears in two of their tables (a forked or prefix-cached prompt block
 * shows up in every sequence that holds it), else 0.  Blocks shared only
 * with sequences outside the call do not count: the hint is about reads
 * within one call. */
int pkv_bm_blocks_unshared(const pkv_block_manager* bm, const int32_t* seqs,
                           int32_t n, int32_t* unshared);

typedef struct pkv_bm_stats {
  int64_t free_blocks;     /* blocks with no reference (the free list, and
                              with prefix caching the evictable blocks)     */
  int64_t used_blocks;     /* blocks held by at least one sequence          */
  int64_t shared_blocks;   /* blocks held by more than one sequence         */
  int64_t live_sequences;
  int64_t logical_tokens;  /* sum of the live sequences' lengths            */
  int64_t stored_tokens;   /* token slots written in used blocks (a shared
                              block counts once)                            */
  int64_t wasted_slots;    /* used_blocks * block_size - stored_tokens      */
} pkv_bm_stats;

int pkv_bm_get_stats(const pkv_block_manager* bm, pkv_bm_stats* out);

/* Reference count of a physical block (-1 for an id out of range). */
int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);

/* Token count of a sequence (-1 if it is not live). */
int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int32_t seq);

/* ---- the baseline: contiguous reservation of a maximum length ---- */

typedef struct pkv_contig_allocator pkv_contig_allocator;

/* A buffer of num_slots token slots; requests have ids 0 .. max_requests-1. */
pkv_contig_allocator* pkv_ca_create(int64_t num_slots, int32_t max_requests);
void pkv_ca_destroy(pkv_contig_allocator* ca);

/* Reserve num_slots contiguous slots for request req at the lowest-addressed
 * gap that fits (first fit); *start_out gets its first slot.
 * PKV_ERR_NO_BLOCKS when no single gap is large enough, even if the free
 * slots add up to enough (external fragmentation). */
int pkv_ca_reserve(pkv_contig_allocator* ca, int32_t req, int64_t num_slots,
                   int64_t* start_out);

/* Release request req's reservation; adjacent gaps merge. */
int pkv_ca_release(pkv_contig_allocator* ca, int32_t req);

/* Free slots in total, the largest single gap, and the reserved slots. */
int pkv_ca_get_stats(const pkv_contig_allocator* ca, int64_t* free_slots,
                     int64_t* largest_gap, int64_t* reserved_slots);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_BLOCKS_H */
