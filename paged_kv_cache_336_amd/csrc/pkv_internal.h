// pkv_internal.h -- argument blocks and launchers shared between the C-ABI
// layer (pagedkv_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

// Most sequences per call: the tile prefix and the lengths of all sequences
// are held in LDS (8 bytes per sequence).
constexpr int kMaxSeqs = 8192;
constexpr int kMaxSeqsMulti = 4096;  // four LDS words per sequence

// Several query tokens per sequence: the partition kernel's waves are capped
// at 1024 (one per SIMD of a 256-CU part) and a partial slot holds up to four
// 16-column groups, so the workspace stays at 1024 * 2 * 64 columns.
constexpr int kMaxWavesMulti = 1024;
constexpr int kMaxGroupsMulti = 4;

// Column groups per row of paged_attn_multi for these arguments.
int multi_groups_per_row(int q_dtype, int cache_dtype, bool uniform,
                         bool token_scales, int max_query_len, int tpr);

// Most waves of the partition kernel (16 per CU of a 256-CU part); the
// workspace holds two partial slots per wave.
constexpr int kMaxWaves = 4096;

struct AttnArgs {
  float* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* part_o;          // [kMaxWaves][2][slot_heads][D]   partial outputs
  float* part_m;          // [kMaxWaves][2][slot_heads]      running max (log2)
  float* part_l;          // [kMaxWaves][2][slot_heads]      running sum
  int32_t* tile_prefix;   // [num_seqs + 1]  tiles of the sequences before s
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // query heads per kv head
  int32_t group_chunks;   // ceil(group / 16)
  int32_t slot_heads;     // min(16, group): query heads per partial slot
  int32_t block_size;
  int32_t num_blocks;     // table entries are clamped into [0, num_blocks)
  int32_t max_seq_tokens; // max_seq_len: longer lengths are cut to it
  int32_t num_waves;      // waves of the partition kernel's grid
  float qk_scale_log2;    // softmax scale * log2(e)
  int32_t scale_per_head; // fp8 scales: one per kv head (else one per tensor)
  int32_t scale_per_token;  // fp8 scales: k_scale / v_scale are
                            // [num_blocks, block_size, num_kv_heads]
  int32_t kv_stream;      // no block is read by two sequences: streaming loads
  // several query tokens per sequence (paged_attn_multi) only:
  const int32_t* query_start;  // [num_seqs + 1] first query row of each
  int32_t num_query_tokens;    // rows of query / out (starts clamped to it)
  int32_t max_query_len;       // new tokens per sequence at most (clamped)
  int32_t tpr;            // query tokens per 16-column group (16 / group)
  int32_t row_tokens;     // query tokens per row: groups per row * tpr
  int32_t max_rps;        // rows per (sequence, kv head): ceil(max_query_len / row_tokens)
  int64_t query_bytes;    // bytes of the whole query tensor (< 2^31)
  // fused write of each sequence's new token (paged_attn_decode_fused) only:
  const void* new_key;         // [num_seqs, num_kv_heads, head_dim], query type
  const void* new_value;
  const int32_t* slot_mapping; // [num_seqs]; < 0 or >= num_slots: no write
  int64_t num_slots;           // num_blocks * block_size
};

hipError_t launch_attn_multi(const AttnArgs& a, int q_dtype, int cache_dtype,
                             int head_dim, int max_waves, hipStream_t stream);

hipError_t launch_attn_decode(const AttnArgs& a, int q_dtype, int cache_dtype,
                              int head_dim, int max_waves, bool fused_write,
                              hipStream_t stream);

struct WriteArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  const float* k_scale;
  const float* v_scale;
  int64_t num_tokens;
  int64_t num_slots;      // num_blocks * block_size: larger slots are skipped
  int32_t scale_per_head; // fp8 scales: one per kv head (else one per tensor)
  int32_t head_dim;
  int32_t block_size;
  int32_t row_elems;      // num_kv_heads * head_dim
  // per-token fp8 scales: each written (token, kv head) row's own scale is
  // stored here, [num_blocks, block_size, num_kv_heads] (null otherwise)
  float* k_token_scales;
  float* v_token_scales;
};

hipError_t launch_cache_write(const WriteArgs& a, int src_dtype,
                              int cache_dtype, hipStream_t stream);

struct CopyArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* pairs;   // {src, dst} or, with prefix, {src, dst, tokens}
  int64_t num_pairs;
  int64_t num_blocks;     // pairs naming a block outside the pool are skipped
  int64_t block_bytes;
  int64_t token_bytes;    // one token's rows of all kv heads
  int32_t block_size;
  int32_t prefix;         // 1: copy only the first `tokens` token rows
  int32_t num_layers;     // pools of every layer, layer_stride bytes apart
  int64_t layer_stride;
  int32_t piece_bytes;    // 16 (pools) or 4 (per-token scale arrays)
};

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

}  // namespace pkv
