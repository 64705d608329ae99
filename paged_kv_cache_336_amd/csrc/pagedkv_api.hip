// pagedkv_api.hip -- the C ABI declared in include/pagedkv.h: argument
// validation (before any HIP call), workspace layout, launch sizing and
// dispatch to the kernels in attn_decode.hip and cache_ops.hip.

#include <limits.h>

#include "pkv_internal.h"

using namespace pkv;

namespace {

bool valid_dtype(int d) {
  return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16 || d == PKV_FP8_E4M3;
}

int dtype_bytes(int d) {
  return d == PKV_F32 ? 4 : (d == PKV_FP8_E4M3 ? 1 : 2);
}

bool aligned(const void* p, uintptr_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

// Partition choice when the caller passes 0: about 4096 workgroups (16 per
// CU of a 256-CU part) if every sequence were max_seq_len long, in multiples
// of 128 tokens (one 32-token tile for each of a workgroup's 4 waves),
// between 128 and 512 tokens so a partition stays a few microseconds of work
// and the partials stay a few percent of the K/V bytes.
int32_t auto_partition(int64_t units_per_token_range, int32_t max_seq_len) {
  const int64_t target_workgroups = 4096;
  int64_t p = (int64_t)max_seq_len * units_per_token_range / target_workgroups;
  p = (p + 127) / 128 * 128;
  if (p < 128) p = 128;
  if (p > 512) p = 512;
  return (int32_t)p;
}

struct AttnShape {
  int32_t partition;
  int32_t max_parts;
  int32_t group;
  int32_t group_chunks;
  size_t ws_bytes;
  size_t off_m, off_l, off_o;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int attn_shape(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
               int32_t head_dim, int32_t max_seq_len, int32_t partition_size,
               AttnShape* out) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_seq_len < 0)
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % 32 != 0 ||
      partition_size > kMaxPartition)
    return PKV_ERR_SHAPE;
  AttnShape s{};
  s.group = num_q_heads / num_kv_heads;
  s.group_chunks = (s.group + 15) / 16;
  const int64_t units = (int64_t)num_seqs * num_kv_heads * s.group_chunks;
  s.partition = partition_size ? partition_size
                               : auto_partition(units, max_seq_len);
  s.max_parts = max_seq_len > 0 ? (max_seq_len + s.partition - 1) / s.partition : 1;
  if (s.max_parts < 1) s.max_parts = 1;
  if (units * s.max_parts > INT_MAX / 64) return PKV_ERR_SHAPE;
  if (s.max_parts > 1) {
    const size_t rows = (size_t)num_seqs * num_q_heads * s.max_parts;
    s.off_m = 0;
    s.off_l = align_up(s.off_m + rows * 4, 256);
    s.off_o = align_up(s.off_l + rows * 4, 256);
    s.ws_bytes = s.off_o + rows * (size_t)head_dim * 4;
  }
  *out = s;
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer";
    case PKV_ERR_SHAPE: return "invalid or inconsistent size";
    case PKV_ERR_DTYPE: return "unsupported dtype or dtype pairing";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int cache_write_slots(const void* key, const void* value, int src_dtype,
                      void* k_cache, void* v_cache, int cache_dtype,
                      const int32_t* slot_mapping, int64_t num_tokens,
                      int64_t num_blocks, int32_t block_size,
                      int32_t num_kv_heads, int32_t head_dim,
                      const float* k_scale, const float* v_scale,
                      hipStream_t stream) {
  if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
  if (src_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (cache_dtype != PKV_FP8_E4M3 && src_dtype != cache_dtype) return PKV_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1)
    return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (num_blocks * (int64_t)block_size > INT_MAX) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
  if (cache_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 4))
    return PKV_ERR_ALIGN;
  WriteArgs a{};
  a.key = key;
  a.value = value;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slot_mapping = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_tokens = num_tokens;
  a.block_size = block_size;
  a.row_elems = num_kv_heads * head_dim;
  return launch_cache_write(a, src_dtype, cache_dtype, stream) == hipSuccess
             ? PKV_OK : PKV_ERR_HIP;
}

int copy_blocks(void* k_cache, void* v_cache, int cache_dtype,
                const int32_t* block_pairs, int64_t num_pairs,
                int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                int32_t head_dim, hipStream_t stream) {
  if (!valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
  if (num_pairs < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1)
    return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_pairs) return PKV_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 4))
    return PKV_ERR_ALIGN;
  CopyArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.pairs = block_pairs;
  a.num_pairs = num_pairs;
  a.block_bytes = (int64_t)block_size * num_kv_heads * head_dim *
                  dtype_bytes(cache_dtype);
  return launch_copy_blocks(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int32_t paged_attn_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t max_seq_len,
                                  int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_seq_len < 0 ||
      num_q_heads % num_kv_heads != 0 || partition_size < 0 ||
      partition_size % 32 != 0 || partition_size > kMaxPartition)
    return -PKV_ERR_SHAPE;
  if (partition_size) return partition_size;
  const int32_t g = num_q_heads / num_kv_heads;
  return auto_partition((int64_t)num_seqs * num_kv_heads * ((g + 15) / 16),
                        max_seq_len);
}

size_t paged_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t partition_size) {
  AttnShape s;
  if (attn_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                 partition_size, &s) != PKV_OK)
    return (size_t)-1;
  return s.ws_bytes;
}

int paged_attn_decode(float* out, const void* query, int q_dtype,
                      const void* k_cache, const void* v_cache,
                      int cache_dtype, const float* k_scale,
                      const float* v_scale, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens,
                      int32_t max_seq_len, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_blocks,
                      int32_t block_size, float scale,
                      int32_t partition_size, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return PKV_ERR_DTYPE;
  if (q_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (cache_dtype != PKV_FP8_E4M3 && q_dtype != cache_dtype) return PKV_ERR_DTYPE;
  if (num_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1)
    return PKV_ERR_SHAPE;
  if (num_blocks * (int64_t)block_size > INT_MAX) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return PKV_ERR_SHAPE;
  AttnShape s;
  const int rc = attn_shape(num_seqs, num_q_heads, num_kv_heads, head_dim,
                            max_seq_len, partition_size, &s);
  if (rc != PKV_OK) return rc;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens)
    return PKV_ERR_NULL;
  if (cache_dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return PKV_ERR_ALIGN;
  if (s.ws_bytes > 0) {
    if (!workspace || workspace_bytes < s.ws_bytes) return PKV_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PKV_ERR_ALIGN;
  }
  AttnArgs a{};
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.part_m = s.ws_bytes ? reinterpret_cast<float*>(ws + s.off_m) : nullptr;
  a.part_l = s.ws_bytes ? reinterpret_cast<float*>(ws + s.off_l) : nullptr;
  a.part_o = s.ws_bytes ? reinterpret_cast<float*>(ws + s.off_o) : nullptr;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = s.group;
  a.group_chunks = s.group_chunks;
  a.block_size = block_size;
  a.partition_size = s.partition;
  a.max_parts = s.max_parts;
  a.qk_scale_log2 = scale * 1.4426950408889634f;
  const int grid = num_seqs * num_kv_heads * s.group_chunks * s.max_parts;
  return launch_attn_decode(a, q_dtype, cache_dtype, head_dim, grid, stream) ==
                 hipSuccess
             ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
