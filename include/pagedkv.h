/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV-cache hot path.
 *
 * Three operations, all asynchronous on the caller's HIP stream:
 *
 *   cache_write_slots  slot-mapped scatter of new key/value rows into the
 *                      paged pools ("How PagedAttention Works in vLLM ...",
 *                      instagit.com, section "write_to_paged_cache: Direct
 *                      In-Place Updates", and its code example);
 *   copy_blocks        whole-block copies for copy-on-write ("PagedAttention",
 *                      shubhamtatvamasi.com, section "Sharing and
 *                      copy-on-write" and the FAQ entry on copy-on-write for
 *                      parallel sampling), and copy_block_prefixes, which
 *                      copies only the tokens a block holds;
 *   paged_attn_decode  one decode query per sequence attends over its tokens
 *                      by walking its block table over the shared pool
 *                      ("PagedAttention", section "How attention reads paged
 *                      memory"), with an online softmax over each wave's
 *                      share of the sequence and a log-sum-exp merge of the
 *                      shares of a sequence split between waves.
 *
 * Memory layout (all buffers are device memory owned by the caller):
 *   k_cache, v_cache   [num_blocks, block_size, num_kv_heads, head_dim],
 *                      contiguous, one pool per tensor (the "flash" layout's
 *                      kv[0] and kv[1] are exactly this);
 *   block_tables       int32 [num_seqs, max_blocks_per_seq], row-major;
 *                      entry i of row s is the physical block of logical
 *                      block i; only the first ceil(seq_len/block_size)
 *                      entries of a row are read;
 *   seq_lens           int32 [num_seqs]: tokens of the sequence, including
 *                      the one written this step;
 *   slot_mapping       int32 [num_tokens]: slot = block * block_size + offset;
 *                      a negative slot skips the token;
 *   query, out         [num_seqs, num_q_heads, head_dim]; out is float32;
 *                      query head q reads cache head q / (num_q_heads /
 *                      num_kv_heads);
 *   k_scale, v_scale   float32 scalars in device memory, read only for an
 *                      fp8 cache (stored value = decode(code) * scale).
 *
 * Errors: every host-checkable precondition is checked before any HIP call;
 * a failed check returns a non-zero pkv_status and launches nothing.  The
 * contents of device buffers (table entries in range, slots in range,
 * lengths within the table's reach, no duplicate slots, copy pairs with
 * distinct destinations that are not also sources) are the caller's
 * contract, verified only in debug mode (pkv_set_debug_checks,
 * PAGEDKV_DEBUG=1: PKV_ERR_RANGE).  Breaking it gives unspecified results
 * but never an access outside the buffers: table entries outside
 * [0, num_blocks) are clamped into the pool, slots and copy pairs outside it
 * are skipped, lengths are cut to max_seq_len, and query extents
 * (paged_attn_multi) to the query rows there are.  A failed launch returns
 * PKV_ERR_HIP.  The library allocates no memory, never synchronises
 * (outside debug mode) and keeps no state beyond cached launch sizes and
 * the debug setting: calls are thread-safe, and two calls that share an
 * attention workspace must not overlap in time.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PKV_FP8_E4M3 is the OCP E4M3 "fn" format (bias 7, no
 * infinities, S.1111.111 = NaN, largest magnitude 448); PKV_FP8_E5M2 the OCP
 * E5M2 format (bias 15, IEEE infinities and NaNs, largest finite magnitude
 * 57344).
 *
 * An fp8 cache's values are stored over scales: a cache dtype argument of
 * PKV_FP8_E4M3 or PKV_FP8_E5M2 takes k_scale / v_scale as one float32 each;
 * OR-ing in PKV_SCALE_PER_HEAD takes them as float32 [num_kv_heads], one per
 * kv head; OR-ing in PKV_SCALE_PER_TOKEN takes them as float32 [num_blocks,
 * block_size, num_kv_heads] arrays laid out like the pools without the
 * head_dim axis: one scale per (token slot, kv head), written beside each
 * row by cache_write_slots_token_scaled and carried through copies by
 * copy_token_scales.  (The copy calls accept, and ignore, both flags.)
 * The pages' scale is one per tensor ("How PagedAttention Works in vLLM
 * ...", instagit.com, section "write_to_paged_cache": k_scale / v_scale
 * with the cache dtype); the per-head and per-token layouts generalise it. */
typedef enum pkv_dtype {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3,
  PKV_FP8_E5M2 = 4
} pkv_dtype;

#define PKV_SCALE_PER_HEAD 0x100
#define PKV_SCALE_PER_TOKEN 0x200

/* Cache-policy hint, OR-ed into any call's cache dtype argument: the caller
 * states that no physical block is read by more than one sequence of the
 * call (no shared prefix, no forked samples).  paged_attn_decode,
 * paged_attn_decode_fused and paged_attn_multi (its per-wave rows; the
 * workgroup rows of long query runs share tiles through LDS and ignore it)
 * then fetch V rows of 128 bytes or more (head_dim * element size) with
 * non-temporal loads, which measured faster
 * on such batches; without the hint the rows go through the caches, so a
 * block shared by several sequences is served from them after its first
 * read (the pages' copy-on-write sharing: "PagedAttention",
 * shubhamtatvamasi.com, section "Sharing and copy-on-write").  The hint
 * changes no result, only speed, and is wrong-but-harmless if untrue (shared
 * blocks are then re-read from HBM).  The other calls accept and ignore it. */
#define PKV_KV_STREAM 0x400

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                   */
  PKV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent       */
  PKV_ERR_DTYPE = 3,       /* unknown dtype or unsupported dtype pairing   */
  PKV_ERR_UNSUPPORTED = 4, /* valid request the library does not implement */
  PKV_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned             */
  PKV_ERR_WORKSPACE = 6,   /* attention workspace missing or too small     */
  PKV_ERR_RANGE = 7,       /* debug checks: device contents break the call's
                              contract (see pkv_set_debug_checks)          */
  PKV_ERR_HIP = 8,         /* the HIP runtime reported an error            */
  PKV_ERR_NO_BLOCKS = 9,   /* block manager: too few free blocks or slots  */
  PKV_ERR_SEQ = 10         /* block manager: sequence not live / in use    */
} pkv_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* pkv_status_string(int status);

/*
 * pkv_set_debug_checks -- turn the checks of device contents on (non-zero)
 * or off (0) for every later call in the process; returns the previous
 * setting.  The initial setting is read once, at the first call that needs
 * it, from the environment: PAGEDKV_DEBUG set to anything but "" or "0"
 * turns the checks on.
 *
 * With the checks on, every device call first copies the small index
 * arrays it was given (block tables, lengths, query starts, slots, copy
 * pairs) to the host on its stream, waits for the copy (so the call is no
 * longer asynchronous), and verifies the contract stated for the call:
 *   lengths         0 <= seq_lens[s] <= max_seq_len;
 *   block tables    the first ceil(seq_lens[s] / block_size) entries of row
 *                   s lie in [0, num_blocks);
 *   slots           every slot >= 0 is below num_blocks * block_size, and
 *                   no slot >= 0 appears twice (a slot names one token's
 *                   place: "How PagedAttention Works in vLLM ...",
 *                   instagit.com, section "write_to_paged_cache");
 *   fused slots     additionally, slot s >= 0 is that of position
 *                   seq_lens[s] - 1 through row s of the table;
 *   copy pairs      src and dst in [0, num_blocks), destinations distinct,
 *                   no destination also a source (a copy-on-write copies a
 *                   shared block into a fresh one before the write:
 *                   "PagedAttention", shubhamtatvamasi.com, FAQ entry on
 *                   copy-on-write);
 *   query starts    non-decreasing from >= 0 to <= num_query_tokens, each
 *                   sequence's count <= max_query_len and <= its length.
 * A violation returns PKV_ERR_RANGE and launches nothing; a failed copy
 * returns PKV_ERR_HIP.  With the checks off (the default) nothing is copied
 * and the calls are as fast as without this facility.
 */
int pkv_set_debug_checks(int enable);

/*
 * cache_write_slots -- write new K/V rows into the pools in place.
 *
 * key, value   [num_tokens, num_kv_heads, head_dim] of src_dtype, contiguous.
 * k_cache,
 * v_cache      pools of cache_dtype (layout above), updated in place.
 * slot_mapping device int32 [num_tokens]; token t goes to block
 *              slot/block_size, offset slot%block_size; slot < 0 skips it.
 * k_scale,
 * v_scale      device float32 scales (one, or [num_kv_heads] with
 *              PKV_SCALE_PER_HEAD), required for an fp8 cache, ignored
 *              otherwise.
 *
 * Element conversion: with src_dtype == cache_dtype the row is copied bit for
 * bit.  With an fp8 cache (src_dtype F32, F16 or BF16) element [h, d] of a
 * row is encoded as enc(float32(x) / scale_h): IEEE float32 division, round
 * to nearest even; for E4M3 finite values beyond 448 saturate to +-448, for
 * E5M2 magnitudes from 61440 on become infinity (IEEE overflow); NaN stays
 * NaN.  No other pairing is accepted (PKV_ERR_DTYPE).  num_tokens == 0 is a valid
 * no-op.  head_dim must be 64 or 128; pointers 16-byte aligned.  Per-token
 * scales (PKV_SCALE_PER_TOKEN) are written by cache_write_slots_token_scaled
 * only (PKV_ERR_DTYPE here).
 */
int cache_write_slots(const void* key, const void* value, int src_dtype,
                      void* k_cache, void* v_cache, int cache_dtype,
                      const int32_t* slot_mapping, int64_t num_tokens,
                      int64_t num_blocks, int32_t block_size,
                      int32_t num_kv_heads, int32_t head_dim,
                      const float* k_scale, const float* v_scale,
                      hipStream_t stream);

/*
 * cache_write_slots_token_scaled -- cache_write_slots into an fp8 cache with
 * a scale per written row: each (token, kv head) row of key and value gets
 * its own scale, the largest magnitude of the row (NaN elements left out)
 * over the format's largest finite value (448 for E4M3, 57344 for E5M2) as
 * an IEEE float32 division, or 1 for a row with no nonzero element; the row
 * is encoded over that scale as by cache_write_slots (its largest element
 * lands on the largest finite code), and the scale is stored at
 * [slot / block_size, slot % block_size, head] of k_scales / v_scales.
 * (The pages scale per tensor, "How PagedAttention Works in vLLM ...",
 * instagit.com, section "write_to_paged_cache"; a scale per row keeps one
 * large row from coarsening the codes of all others.)
 *
 * cache_dtype   PKV_FP8_E4M3 or PKV_FP8_E5M2, with or without
 *               PKV_SCALE_PER_TOKEN (anything else: PKV_ERR_DTYPE).
 * k_scales,
 * v_scales      device float32 [num_blocks, block_size, num_kv_heads],
 *               4-byte aligned; only the written slots' entries change.
 * Other arguments and rules as cache_write_slots.
 */
int cache_write_slots_token_scaled(const void* key, const void* value,
                                   int src_dtype, void* k_cache,
                                   void* v_cache, int cache_dtype,
                                   float* k_scales, float* v_scales,
                                   const int32_t* slot_mapping,
                                   int64_t num_tokens, int64_t num_blocks,
                                   int32_t block_size, int32_t num_kv_heads,
                                   int32_t head_dim, hipStream_t stream);

/*
 * copy_token_scales, copy_token_scale_prefixes -- the per-token scale
 * arrays (float32 [num_blocks, block_size, num_kv_heads], 4-byte aligned)
 * through the copies copy_blocks / copy_block_prefixes make of the pools:
 * the same pairs {src, dst} (whole blocks) or triples {src, dst, tokens}
 * (slots 0 .. tokens-1, tokens clamped to [0, block_size]), with the same
 * rules.  A copy-on-write of a per-token-scaled fp8 cache calls both.
 */
int copy_token_scales(float* k_scales, float* v_scales,
                      const int32_t* block_pairs, int64_t num_pairs,
                      int64_t num_blocks, int32_t block_size,
                      int32_t num_kv_heads, hipStream_t stream);
int copy_token_scale_prefixes(float* k_scales, float* v_scales,
                              const int32_t* block_triples,
                              int64_t num_copies, int64_t num_blocks,
                              int32_t block_size, int32_t num_kv_heads,
                              hipStream_t stream);

/*
 * copy_blocks -- for each pair (src, dst), every slot of block dst in both
 * pools takes the bytes of block src.
 *
 * block_pairs  device int32 [num_pairs][2] = {src, dst}.  Destinations must be
 *              distinct and no destination may also be a source (otherwise
 *              the result depends on scheduling).  num_pairs == 0 is a valid
 *              no-op (nothing is launched).
 */
int copy_blocks(void* k_cache, void* v_cache, int cache_dtype,
                const int32_t* block_pairs, int64_t num_pairs,
                int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                int32_t head_dim, hipStream_t stream);

/*
 * copy_block_prefixes -- copy-on-write of the tokens a block already holds
 * ("PagedAttention", shubhamtatvamasi.com, FAQ entry on copy-on-write for
 * parallel sampling: the engine copies the existing tokens into the new
 * block).  For each triple {src, dst, tokens}, slots 0 .. tokens-1 of block
 * dst in both pools take the bytes of the same slots of block src; slots from
 * tokens on are left as they are.  tokens is clamped to [0, block_size].
 *
 * block_triples  device int32 [num_copies][3].  The same rules as
 *                copy_blocks otherwise (distinct destinations that are not
 *                sources; num_copies == 0 is a no-op).
 */
int copy_block_prefixes(void* k_cache, void* v_cache, int cache_dtype,
                        const int32_t* block_triples, int64_t num_copies,
                        int64_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim,
                        hipStream_t stream);

/*
 * copy_blocks_layers, copy_block_prefixes_layers -- the same copies in the
 * pools of every layer of a model, in one launch.  A block id names the same
 * block in every layer ("PagedAttention", shubhamtatvamasi.com, the table in
 * "The idea: page the KV cache": a KV block is 16 tokens x all layers' K and
 * V), so a copy-on-write copies it in each layer's pools.
 *
 * k_caches,
 * v_caches      the first layer's pools; layer l's are layer_stride bytes
 *               further on (e.g. one allocation [num_layers, num_blocks,
 *               block_size, num_kv_heads, head_dim] per cache); layer_stride
 *               a multiple of 16, at least one pool's bytes when
 *               num_layers > 1 (layers must not overlap).
 * num_layers    1 .. 65535.
 * Other arguments, and the result in each layer, as copy_blocks /
 * copy_block_prefixes.
 */
int copy_blocks_layers(void* k_caches, void* v_caches, int64_t layer_stride,
                       int32_t num_layers, int cache_dtype,
                       const int32_t* block_pairs, int64_t num_pairs,
                       int64_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim,
                       hipStream_t stream);
int copy_block_prefixes_layers(void* k_caches, void* v_caches,
                               int64_t layer_stride, int32_t num_layers,
                               int cache_dtype, const int32_t* block_triples,
                               int64_t num_copies, int64_t num_blocks,
                               int32_t block_size, int32_t num_kv_heads,
                               int32_t head_dim, hipStream_t stream);

/*
 * paged_attn_workspace_size -- bytes of device workspace paged_attn_decode
 * needs for these arguments, or (size_t)-1 for invalid arguments.
 *
 * The workspace carries, from the first to the second kernel of one call, the
 * per-sequence tile prefix and the partial results (running max, running sum
 * and unnormalised output of every query head) of the rows whose tiles are
 * split between waves.  It needs no initialisation and may be reused by later
 * calls of any shape that fit its size (the size depends only on these
 * arguments: about 2 * 4096 * min(16, Hq/Hkv) * (head_dim + 2) * 4 bytes).
 */
size_t paged_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim);

/*
 * paged_attn_decode -- out[s, q, :] = softmax(scale * q . K_s^T) V_s over
 * tokens 0 .. seq_lens[s]-1 of sequence s, gathered through its block table.
 *
 * query        [num_seqs, num_q_heads, head_dim] of q_dtype, contiguous.
 * out          float32 [num_seqs, num_q_heads, head_dim].
 * k_cache,
 * v_cache      pools of cache_dtype; (q_dtype, cache_dtype) is one of
 *              (F32,F32) (F16,F16) (BF16,BF16) or (F32|F16|BF16, FP8_E4M3|
 *              FP8_E5M2).
 * k_scale,
 * v_scale      device float32 scales, required for an fp8 cache: one each,
 *              [num_kv_heads] with PKV_SCALE_PER_HEAD, or the per-token
 *              arrays [num_blocks, block_size, num_kv_heads] with
 *              PKV_SCALE_PER_TOKEN (token t of a sequence is then read as
 *              decode(code) * its own scale, in its score and in its share
 *              of the value sum).
 * max_seq_len  host-side upper bound of seq_lens (a sequence longer than it
 *              is the caller's error: it is cut to max_seq_len).
 * scale        softmax scale applied to q . k.
 * max_waves    0 to spread the work over every wave the GPU holds at once,
 *              else at most this many (rounded down to a multiple of 4).
 *              All 32-token tiles of all (sequence, kv head) rows are divided
 *              into equal contiguous shares, one per wave; a row split
 *              between waves is merged by log-sum-exp, giving the same result
 *              up to float32 rounding for any split (and the same bits on
 *              every run of one call).
 * workspace    device buffer of workspace_bytes >= paged_attn_workspace_size,
 *              256-byte aligned.
 *
 * Two kernels are launched on the stream (tiles, then the merge of split
 * rows).  At most 8192 sequences per call (PKV_ERR_UNSUPPORTED beyond).
 * A sequence of length 0 yields zeros.  num_q_heads must be a multiple of
 * num_kv_heads; head_dim 64 or 128; max_blocks_per_seq * block_size >=
 * max_seq_len.  Pointers 16-byte aligned (seq_lens, block_tables: 4-byte).
 */
int paged_attn_decode(float* out, const void* query, int q_dtype,
                      const void* k_cache, const void* v_cache,
                      int cache_dtype, const float* k_scale,
                      const float* v_scale, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                      int32_t max_seq_len, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_blocks,
                      int32_t block_size, float scale, int32_t max_waves,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * call allocates nothing; the partial results that paged_attn_decode keeps
 * in the caller's workspace live in a device array of the library instead
 * (16.3 MiB per GPU the library runs on, held until the process ends; its
 * device address is looked up once per device, at the first call there).
 *
 * Arguments, results and rules are paged_attn_decode's, with these limits:
 * the split uses at most 1024 waves (max_waves 0 means every wave the GPU
 * holds at once, up to 1024; max_waves above 1024 returns
 * PKV_ERR_UNSUPPORTED), and the debug checks of pkv_set_debug_checks are
 * not run (they copy and wait).  On a GPU whose resident waves number 1024
 * or fewer (an MI355X holds 1024 in this kernel's launch shape) the output
 * is that of paged_attn_decode with the same max_waves, bit for bit.
 *
 * Every call on one GPU shares that GPU's array and needs nothing in it
 * from an earlier call (no part of it must start at zero).  Calls that
 * overlap in time on one GPU (on different streams, or from different
 * threads without ordering) race on it and give unspecified results;
 * calls on one stream never overlap.
 */
int paged_attn_decode_noalloc(float* out, const void* query, int q_dtype,
                              const void* k_cache, const void* v_cache,
                              int cache_dtype, const float* k_scale,
                              const float* v_scale,
                              const int32_t* block_tables,
                              int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t max_seq_len,
                              int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim,
                              int64_t num_blocks, int32_t block_size,
                              float scale, int32_t max_waves,
                              hipStream_t stream);

/*
 * paged_attn_decode_fused -- cache_write_slots of one new token per sequence
 * and paged_attn_decode in one launch: the result (out and both pools) is
 * that of cache_write_slots(key, value, ..., slot_mapping, num_seqs, ...)
 * followed by paged_attn_decode(...), bit for bit.  The pages' step is
 * "write the new token's key and value into its slot, then attend over the
 * sequence through its block table" ("How PagedAttention Works in vLLM ...",
 * instagit.com, section "write_to_paged_cache"; "PagedAttention",
 * shubhamtatvamasi.com, section "How attention reads paged memory"); here
 * the wave that reads a sequence's last tile for a kv head writes that head's
 * new row first.
 *
 * key, value    [num_seqs, num_kv_heads, head_dim] of q_dtype (for an fp8
 *               cache the new rows are encoded e4m3(x / scale) as by
 *               cache_write_slots; otherwise q_dtype == cache_dtype).
 * slot_mapping  int32 [num_seqs]: the slot of position seq_lens[s] - 1 of
 *               sequence s (block * block_size + offset, through its table),
 *               or negative to write nothing for s.  A slot elsewhere is the
 *               caller's error (unspecified values, no access outside the
 *               pools; slots outside the pool are skipped).
 * Other arguments as paged_attn_decode (same workspace).  At most 16 query
 * heads per kv head (PKV_ERR_UNSUPPORTED beyond): each kv head's last tile is
 * then read by exactly the wave that writes it.  Per-token scales are not
 * written here (PKV_ERR_UNSUPPORTED): use cache_write_slots_token_scaled and
 * paged_attn_decode.  When the batch has more
 * (sequence, kv head) rows than the GPU holds waves, the write goes as its
 * own launch ahead of the attention (faster there; the same result).
 */
int paged_attn_decode_fused(float* out, const void* query, int q_dtype,
                            const void* key, const void* value,
                            void* k_cache, void* v_cache, int cache_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* slot_mapping,
                            const int32_t* block_tables,
                            int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t max_seq_len,
                            int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int64_t num_blocks, int32_t block_size,
                            float scale, int32_t max_waves, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attn_multi_workspace_size -- bytes of device workspace
 * paged_attn_multi needs for these arguments, or (size_t)-1 for invalid ones
 * (about 2 * 4096 * 16 * (head_dim + 2) * 4 bytes).  Same contract as
 * paged_attn_workspace_size.
 */
size_t paged_attn_multi_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim);

/*
 * paged_attn_multi -- paged attention for several new query tokens per
 * sequence: a chunk of a prompt attending to its cached prefix, or the draft
 * tokens of a speculative decoder being verified.  The read path of
 * "PagedAttention" (shubhamtatvamasi.com, section "How attention reads paged
 * memory") with the causal rule of decoder attention among the new tokens:
 * sequence s holds seq_lens[s] = L tokens (the new ones included, their keys
 * and values already written, e.g. by cache_write_slots), its last
 * q = query_start[s+1] - query_start[s] tokens are new, and new token j
 * (position L - q + j) attends to tokens 0 .. L - q + j:
 *
 *   out[query_start[s] + j, h, :] =
 *       softmax(scale * query[query_start[s] + j, h] . K_s[0 .. L-q+j]^T)
 *       V_s[0 .. L-q+j]
 *
 * query        [num_query_tokens, num_q_heads, head_dim] of q_dtype, the new
 *              tokens sequence after sequence.
 * out          float32 [num_query_tokens, num_q_heads, head_dim]; rows that
 *              belong to no sequence are left as they are.
 * query_start  int32 [num_seqs + 1], non-decreasing, query_start[0] >= 0,
 *              query_start[num_seqs] <= num_query_tokens, and q <= L for
 *              every sequence.
 * max_query_len  host-side upper bound of q over the sequences
 *              (<= max_seq_len).
 * The remaining arguments are those of paged_attn_decode; with one new token
 * per sequence (query_start[s] = s) the result is paged_attn_decode's, bit
 * for bit.
 *
 * Work split: the 16 query columns of an MFMA tile (a group) hold 16 / G new
 * tokens of all G = num_q_heads / num_kv_heads heads of one kv head, and a
 * row of NG groups reads a sequence's keys and values once for its
 * NG * 16 / G new tokens: NG = 1 for short runs (drafted tokens), 4 for
 * longer ones, and 8 -- a row per workgroup, the tiles staged through LDS
 * -- when max_query_len fills 12 or more groups on a 16-bit cache that the
 * queries share, with block_size % 16 == 0 and no per-token scales.  All
 * 32-token tiles of all rows are divided evenly among the waves (or
 * workgroups) and split rows are merged by log-sum-exp, as in
 * paged_attn_decode.  At most 4096 sequences and G <= 16
 * (PKV_ERR_UNSUPPORTED beyond); the query tensor below 2 GiB and
 * num_seqs * num_kv_heads * ceil(max_query_len / (NG * 16 / G)) *
 * ceil(max_seq_len / 32) < 2^31 (PKV_ERR_SHAPE beyond).  A call with no query
 * token launches nothing.
 */
int paged_attn_multi(float* out, const void* query, int q_dtype,
                     const void* k_cache, const void* v_cache, int cache_dtype,
                     const float* k_scale, const float* v_scale,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, const int32_t* query_start,
                     int32_t num_query_tokens, int32_t max_query_len,
                     int32_t max_seq_len, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int64_t num_blocks, int32_t block_size,
                     float scale, int32_t max_waves, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
