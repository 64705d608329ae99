// pkv_internal.h -- argument blocks and launchers shared between the C-ABI
// layer (pagedkv_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

// Longest partition (tokens).  With block_size % 16 == 0 a partition of at
// most this many tokens starting at a multiple of 32 touches at most
// kMaxTableWindow blocks (bs 16: exactly P/16; bs >= 32: at most P/32 + 2).
constexpr int kMaxPartition = 4096;
constexpr int kMaxTableWindow = kMaxPartition / 16;

struct AttnArgs {
  float* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* part_o;          // [S, Hq, max_parts, D]
  float* part_m;          // [S, Hq, max_parts]  running max (log2 domain)
  float* part_l;          // [S, Hq, max_parts]  running sum
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // query heads per kv head
  int32_t group_chunks;   // ceil(group / 16)
  int32_t block_size;
  int32_t partition_size;
  int32_t max_parts;
  float qk_scale_log2;    // softmax scale * log2(e)
};

hipError_t launch_attn_decode(const AttnArgs& a, int q_dtype, int cache_dtype,
                              int head_dim, int grid, hipStream_t stream);

struct WriteArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  const float* k_scale;
  const float* v_scale;
  int64_t num_tokens;
  int32_t block_size;
  int32_t row_elems;      // num_kv_heads * head_dim
};

hipError_t launch_cache_write(const WriteArgs& a, int src_dtype,
                              int cache_dtype, hipStream_t stream);

struct CopyArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* pairs;
  int64_t num_pairs;
  int64_t block_bytes;
};

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

}  // namespace pkv
