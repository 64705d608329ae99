// pagedkv_api.hip -- the C ABI declared in include/pagedkv.h: argument
// validation (before any HIP call), workspace layout, launch sizing and
// dispatch to the kernels in attn_decode.hip, attn_multi.hip and
// cache_ops.hip.

#include <limits.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

using namespace pkv;

namespace {

bool valid_dtype(int d) {
  return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16 || d == PKV_FP8_E4M3 ||
         d == PKV_FP8_E5M2;
}

bool is_fp8_dtype(int d) { return d == PKV_FP8_E4M3 || d == PKV_FP8_E5M2; }

int dtype_bytes(int d) {
  return d == PKV_F32 ? 4 : (is_fp8_dtype(d) ? 1 : 2);
}

// A cache dtype argument: the dtype code, optionally OR-ed with one fp8
// scale layout flag (per kv head or per token; fp8 caches only) and with the
// PKV_KV_STREAM hint (any cache; *kv_stream, when asked for).  Any other bit
// is an error.  Returns false if invalid.
bool split_cache_dtype(int arg, int* dtype, bool* per_head, bool* per_token,
                       bool* kv_stream = nullptr) {
  *dtype = arg & 0xFF;
  *per_head = (arg & PKV_SCALE_PER_HEAD) != 0;
  *per_token = (arg & PKV_SCALE_PER_TOKEN) != 0;
  if (kv_stream) *kv_stream = (arg & PKV_KV_STREAM) != 0;
  if ((arg & ~(0xFF | PKV_SCALE_PER_HEAD | PKV_SCALE_PER_TOKEN |
               PKV_KV_STREAM)) != 0)
    return false;
  if (!valid_dtype(*dtype) || (*per_head && *per_token)) return false;
  return !(*per_head || *per_token) || is_fp8_dtype(*dtype);
}

bool aligned(const void* p, uintptr_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

struct AttnShape {
  int32_t group;
  int32_t group_chunks;
  int32_t slot_heads;
  size_t ws_bytes;
  size_t off_m, off_l, off_o;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace: tile prefix [num_seqs + 1] int32 | part_m | part_l | part_o,
// each 256-byte aligned; two partial slots of slot_heads query columns per
// wave.  One query token per sequence: a slot holds up to 16 query heads of
// one kv head.  Several (multi): a slot holds up to four column groups of
// 16 / group tokens times the group's heads (group <= 16), for at most
// kMaxWavesMulti waves.
int attn_shape(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
               int32_t head_dim, bool multi, AttnShape* out,
               int waves_cap = kMaxWaves) {
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1) return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (num_seqs > (multi ? kMaxSeqsMulti : kMaxSeqs)) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  AttnShape s{};
  s.group = num_q_heads / num_kv_heads;
  if (multi && s.group > 16) return PKV_ERR_UNSUPPORTED;
  s.group_chunks = (s.group + 15) / 16;
  s.slot_heads = multi ? 16 / s.group * s.group : (s.group < 16 ? s.group : 16);
  const size_t slots =
      multi ? (size_t)kMaxWavesMulti * 2 * kMaxGroupsMulti * s.slot_heads
            : (size_t)waves_cap * 2 * s.slot_heads;
  s.off_m = align_up((size_t)(num_seqs + 1) * 4, 256);
  s.off_l = align_up(s.off_m + slots * 4, 256);
  s.off_o = align_up(s.off_l + slots * 4, 256);
  s.ws_bytes = s.off_o + slots * (size_t)head_dim * 4;
  *out = s;
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// Scratch of paged_attn_decode_noalloc: the attention workspace of a call
// with at most kScratchWaves waves, held in a device array of this library
// (one per GPU, alive until the process ends) instead of a buffer the
// caller allocates.  Its size is the workspace layout's largest case:
// kMaxSeqs + 1 tile-prefix words, then running maxima and sums and partial
// outputs of 16 query heads per slot at head_dim 128 (16.3 MiB).
// ---------------------------------------------------------------------------
constexpr int kScratchWaves = 1024;
constexpr size_t kScratchSlots = (size_t)kScratchWaves * 2 * 16;
constexpr size_t kScratchOffM = ((size_t)(kMaxSeqs + 1) * 4 + 255) / 256 * 256;
constexpr size_t kScratchOffL = (kScratchOffM + kScratchSlots * 4 + 255) / 256 * 256;
constexpr size_t kScratchOffO = (kScratchOffL + kScratchSlots * 4 + 255) / 256 * 256;
constexpr size_t kScratchBytes = kScratchOffO + kScratchSlots * 128 * 4;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The scratch array's device address on the current device, looked up once
// per device (with that device current) and kept.  The array's name is a
// host-side stand-in in host code: only this address may be handed to
// kernels.
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  const auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return PKV_OK;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
    return PKV_ERR_HIP;
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// Debug checks of device contents (pkv_set_debug_checks, PAGEDKV_DEBUG): the
// index arrays a call was given are copied to the host on the call's stream
// and verified against the call's contract before anything is launched.
// ---------------------------------------------------------------------------
std::atomic<int> g_debug{-1};  // -1: not read from the environment yet

bool debug_checks() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("PAGEDKV_DEBUG");
    int want = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, want);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v > 0;
}

// n int32 values of a device array, on the host (stream-ordered, waited for).
bool fetch_i32(const int32_t* dev, int64_t n, hipStream_t stream,
               std::vector<int32_t>* out) {
  out->assign((size_t)(n > 0 ? n : 0), 0);
  if (n <= 0) return true;
  if (hipMemcpyAsync(out->data(), dev, (size_t)n * sizeof(int32_t),
                     hipMemcpyDeviceToHost, stream) != hipSuccess)
    return false;
  return hipStreamSynchronize(stream) == hipSuccess;
}

// Slots: each one >= 0 below num_slots, and none >= 0 twice.
int check_slots(const std::vector<int32_t>& slots, int64_t num_slots) {
  std::unordered_set<int32_t> seen;
  seen.reserve(slots.size() * 2);
  for (int32_t v : slots) {
    if (v < 0) continue;
    if ((int64_t)v >= num_slots || !seen.insert(v).second) return PKV_ERR_RANGE;
  }
  return PKV_OK;
}

// Copy records {src, dst[, tokens]}: blocks inside the pool, destinations
// distinct, no destination also a source.
int check_copies(const int32_t* records, int64_t n, int width,
                 int64_t num_blocks, hipStream_t stream) {
  std::vector<int32_t> r;
  if (!fetch_i32(records, n * width, stream, &r)) return PKV_ERR_HIP;
  std::unordered_set<int32_t> srcs, dsts;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t src = r[(size_t)(i * width)], dst = r[(size_t)(i * width + 1)];
    if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks)
      return PKV_ERR_RANGE;
    if (!dsts.insert(dst).second) return PKV_ERR_RANGE;
    srcs.insert(src);
  }
  for (int32_t d : dsts)
    if (srcs.count(d)) return PKV_ERR_RANGE;
  return PKV_OK;
}

// Lengths in [0, max_seq_len] and the live table entries inside the pool;
// the host copies of both are returned for further checks.
int check_tables(const int32_t* block_tables, int32_t max_blocks,
                 const int32_t* seq_lens, int32_t num_seqs,
                 int32_t max_seq_len, int64_t num_blocks, int32_t block_size,
                 hipStream_t stream, std::vector<int32_t>* lens,
                 std::vector<int32_t>* tables) {
  if (!fetch_i32(seq_lens, num_seqs, stream, lens) ||
      !fetch_i32(block_tables, (int64_t)num_seqs * max_blocks, stream, tables))
    return PKV_ERR_HIP;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = (*lens)[s];
    if (L < 0 || L > max_seq_len) return PKV_ERR_RANGE;
    const int64_t nblk = ((int64_t)L + block_size - 1) / block_size;
    for (int64_t i = 0; i < nblk; ++i) {
      const int32_t b = (*tables)[(size_t)((int64_t)s * max_blocks + i)];
      if (b < 0 || b >= num_blocks) return PKV_ERR_RANGE;
    }
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_set_debug_checks(int enable) {
  const int prev = debug_checks() ? 1 : 0;
  g_debug.store(enable ? 1 : 0);
  return prev;
}

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer";
    case PKV_ERR_SHAPE: return "invalid or inconsistent size";
    case PKV_ERR_DTYPE: return "unsupported dtype or dtype pairing";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_RANGE:
      return "device contents break the call's contract (debug checks)";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_NO_BLOCKS: return "not enough free blocks";
    case PKV_ERR_SEQ: return "sequence not live, or already live";
  }
  return "unknown status";
}

namespace {

// cache_write_slots (token_scales false: scales read) and
// cache_write_slots_token_scaled (true: each row's scale written to
// k_scales / v_scales).
int write_common(const void* key, const void* value, int src_dtype,
                 void* k_cache, void* v_cache, int cache_dtype,
                 const int32_t* slot_mapping, int64_t num_tokens,
                 int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                 int32_t head_dim, const float* k_scale, const float* v_scale,
                 float* k_scales, float* v_scales, bool token_scales,
                 hipStream_t stream) {
  bool per_head = false, per_token = false;
  const int cache_arg = cache_dtype;
  if (!valid_dtype(src_dtype) ||
      !split_cache_dtype(cache_arg, &cache_dtype, &per_head, &per_token))
    return PKV_ERR_DTYPE;
  // per-token scales are written by the token-scaled call only, which takes
  // an fp8 cache code with or without the per-token flag
  if (token_scales ? (per_head || !is_fp8_dtype(cache_dtype)) : per_token)
    return PKV_ERR_DTYPE;
  if (is_fp8_dtype(src_dtype)) return PKV_ERR_DTYPE;
  if (!is_fp8_dtype(cache_dtype) && src_dtype != cache_dtype) return PKV_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1)
    return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (num_blocks * (int64_t)block_size > INT_MAX) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
  if (token_scales) {
    if (!k_scales || !v_scales) return PKV_ERR_NULL;
    if (!aligned(k_scales, 4) || !aligned(v_scales, 4)) return PKV_ERR_ALIGN;
  } else if (is_fp8_dtype(cache_dtype) && (!k_scale || !v_scale)) {
    return PKV_ERR_NULL;
  }
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 4))
    return PKV_ERR_ALIGN;
  if (debug_checks()) {
    std::vector<int32_t> slots;
    if (!fetch_i32(slot_mapping, num_tokens, stream, &slots)) return PKV_ERR_HIP;
    const int rc = check_slots(slots, num_blocks * (int64_t)block_size);
    if (rc != PKV_OK) return rc;
  }
  WriteArgs a{};
  a.k_token_scales = token_scales ? k_scales : nullptr;
  a.v_token_scales = token_scales ? v_scales : nullptr;
  a.scale_per_head = per_head;
  a.head_dim = head_dim;
  a.key = key;
  a.value = value;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slot_mapping = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_tokens = num_tokens;
  a.num_slots = num_blocks * (int64_t)block_size;
  a.block_size = block_size;
  a.row_elems = num_kv_heads * head_dim;
  return launch_cache_write(a, src_dtype, cache_dtype, stream) == hipSuccess
             ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

int cache_write_slots(const void* key, const void* value, int src_dtype,
                      void* k_cache, void* v_cache, int cache_dtype,
                      const int32_t* slot_mapping, int64_t num_tokens,
                      int64_t num_blocks, int32_t block_size,
                      int32_t num_kv_heads, int32_t head_dim,
                      const float* k_scale, const float* v_scale,
                      hipStream_t stream) {
  return write_common(key, value, src_dtype, k_cache, v_cache, cache_dtype,
                      slot_mapping, num_tokens, num_blocks, block_size,
                      num_kv_heads, head_dim, k_scale, v_scale, nullptr,
                      nullptr, false, stream);
}

int cache_write_slots_token_scaled(const void* key, const void* value,
                                   int src_dtype, void* k_cache,
                                   void* v_cache, int cache_dtype,
                                   float* k_scales, float* v_scales,
                                   const int32_t* slot_mapping,
                                   int64_t num_tokens, int64_t num_blocks,
                                   int32_t block_size, int32_t num_kv_heads,
                                   int32_t head_dim, hipStream_t stream) {
  return write_common(key, value, src_dtype, k_cache, v_cache, cache_dtype,
                      slot_mapping, num_tokens, num_blocks, block_size,
                      num_kv_heads, head_dim, nullptr, nullptr, k_scales,
                      v_scales, true, stream);
}

namespace {

int copy_common(void* k_cache, void* v_cache, int cache_dtype,
                const int32_t* block_pairs, int64_t num_pairs,
                int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                int32_t head_dim, int prefix, int32_t num_layers,
                int64_t layer_stride, hipStream_t stream) {
  bool per_head = false, per_token = false;  // (scales: not in a pool copy)
  const int cache_arg = cache_dtype;
  if (!split_cache_dtype(cache_arg, &cache_dtype, &per_head, &per_token))
    return PKV_ERR_DTYPE;
  if (num_pairs < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1)
    return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  const int64_t pool_bytes = num_blocks * block_size * (int64_t)num_kv_heads *
                             head_dim * dtype_bytes(cache_dtype);
  // the layers' pools must not overlap
  if (num_layers < 1 || num_layers > 65535 ||
      (num_layers > 1 && layer_stride < pool_bytes))
    return PKV_ERR_SHAPE;
  if (num_layers > 1 && layer_stride % 16 != 0) return PKV_ERR_ALIGN;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_pairs) return PKV_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 4))
    return PKV_ERR_ALIGN;
  if (debug_checks()) {
    const int rc = check_copies(block_pairs, num_pairs, prefix ? 3 : 2,
                                num_blocks, stream);
    if (rc != PKV_OK) return rc;
  }
  CopyArgs a{};
  a.num_layers = num_layers;
  a.layer_stride = num_layers > 1 ? layer_stride : 0;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.pairs = block_pairs;
  a.num_pairs = num_pairs;
  a.num_blocks = num_blocks;
  a.token_bytes = (int64_t)num_kv_heads * head_dim * dtype_bytes(cache_dtype);
  a.block_bytes = (int64_t)block_size * a.token_bytes;
  a.block_size = block_size;
  a.prefix = prefix;
  a.piece_bytes = 16;
  return launch_copy_blocks(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// The per-token scale arrays [num_blocks, block_size, num_kv_heads] float32
// through the same copies (one float per thread).
int copy_scales_common(float* k_scales, float* v_scales,
                       const int32_t* records, int64_t num_records,
                       int64_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int prefix, hipStream_t stream) {
  if (num_records < 0 || num_blocks < 1 || block_size < 1 || num_kv_heads < 1)
    return PKV_ERR_SHAPE;
  if (num_blocks * (int64_t)block_size * num_kv_heads > ((int64_t)1 << 40))
    return PKV_ERR_SHAPE;
  if (num_records == 0) return PKV_OK;
  if (!k_scales || !v_scales || !records) return PKV_ERR_NULL;
  if (!aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(records, 4))
    return PKV_ERR_ALIGN;
  if (debug_checks()) {
    const int rc = check_copies(records, num_records, prefix ? 3 : 2,
                                num_blocks, stream);
    if (rc != PKV_OK) return rc;
  }
  CopyArgs a{};
  a.num_layers = 1;
  a.layer_stride = 0;
  a.k_cache = k_scales;
  a.v_cache = v_scales;
  a.pairs = records;
  a.num_pairs = num_records;
  a.num_blocks = num_blocks;
  a.token_bytes = (int64_t)num_kv_heads * 4;
  a.block_bytes = (int64_t)block_size * a.token_bytes;
  a.block_size = block_size;
  a.prefix = prefix;
  a.piece_bytes = 4;
  return launch_copy_blocks(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

int copy_blocks(void* k_cache, void* v_cache, int cache_dtype,
                const int32_t* block_pairs, int64_t num_pairs,
                int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                int32_t head_dim, hipStream_t stream) {
  return copy_common(k_cache, v_cache, cache_dtype, block_pairs, num_pairs,
                     num_blocks, block_size, num_kv_heads, head_dim, 0, 1, 0,
                     stream);
}

int copy_token_scales(float* k_scales, float* v_scales,
                      const int32_t* block_pairs, int64_t num_pairs,
                      int64_t num_blocks, int32_t block_size,
                      int32_t num_kv_heads, hipStream_t stream) {
  return copy_scales_common(k_scales, v_scales, block_pairs, num_pairs,
                            num_blocks, block_size, num_kv_heads, 0, stream);
}

int copy_token_scale_prefixes(float* k_scales, float* v_scales,
                              const int32_t* block_triples,
                              int64_t num_copies, int64_t num_blocks,
                              int32_t block_size, int32_t num_kv_heads,
                              hipStream_t stream) {
  return copy_scales_common(k_scales, v_scales, block_triples, num_copies,
                            num_blocks, block_size, num_kv_heads, 1, stream);
}

int copy_blocks_layers(void* k_caches, void* v_caches, int64_t layer_stride,
                       int32_t num_layers, int cache_dtype,
                       const int32_t* block_pairs, int64_t num_pairs,
                       int64_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim,
                       hipStream_t stream) {
  return copy_common(k_caches, v_caches, cache_dtype, block_pairs, num_pairs,
                     num_blocks, block_size, num_kv_heads, head_dim, 0,
                     num_layers, layer_stride, stream);
}

int copy_block_prefixes_layers(void* k_caches, void* v_caches,
                               int64_t layer_stride, int32_t num_layers,
                               int cache_dtype, const int32_t* block_triples,
                               int64_t num_copies, int64_t num_blocks,
                               int32_t block_size, int32_t num_kv_heads,
                               int32_t head_dim, hipStream_t stream) {
  return copy_common(k_caches, v_caches, cache_dtype, block_triples,
                     num_copies, num_blocks, block_size, num_kv_heads,
                     head_dim, 1, num_layers, layer_stride, stream);
}

int copy_block_prefixes(void* k_cache, void* v_cache, int cache_dtype,
                        const int32_t* block_triples, int64_t num_copies,
                        int64_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim,
                        hipStream_t stream) {
  return copy_common(k_cache, v_cache, cache_dtype, block_triples, num_copies,
                     num_blocks, block_size, num_kv_heads, head_dim, 1, 1, 0,
                     stream);
}

size_t paged_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim) {
  AttnShape s;
  if (attn_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, false, &s) !=
      PKV_OK)
    return (size_t)-1;
  return s.ws_bytes;
}

size_t paged_attn_multi_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads,
                                       int32_t head_dim) {
  AttnShape s;
  if (attn_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, true, &s) !=
      PKV_OK)
    return (size_t)-1;
  return s.ws_bytes;
}

}  // extern "C"

namespace {

// paged_attn_decode and paged_attn_decode_fused: checks, then the launch.
int decode_common(float* out, const void* query, int q_dtype,
                  const void* k_cache, const void* v_cache, int cache_dtype,
                  const float* k_scale, const float* v_scale,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* seq_lens, int32_t max_seq_len,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int64_t num_blocks, int32_t block_size,
                  float scale, int32_t max_waves, void* workspace,
                  size_t workspace_bytes, const void* key, const void* value,
                  const int32_t* slot_mapping, bool fused,
                  hipStream_t stream, bool noalloc = false) {
  bool per_head = false, per_token = false, kv_stream = false;
  const int cache_arg = cache_dtype;
  if (!valid_dtype(q_dtype) ||
      !split_cache_dtype(cache_arg, &cache_dtype, &per_head, &per_token,
                         &kv_stream))
    return PKV_ERR_DTYPE;
  if (is_fp8_dtype(q_dtype)) return PKV_ERR_DTYPE;
  if (!is_fp8_dtype(cache_dtype) && q_dtype != cache_dtype) return PKV_ERR_DTYPE;
  // the fused write stores no per-token scales: write with
  // cache_write_slots_token_scaled, then paged_attn_decode
  if (fused && per_token) return PKV_ERR_UNSUPPORTED;
  if (num_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1 ||
      max_seq_len < 0 || max_waves < 0)
    return PKV_ERR_SHAPE;
  if (num_blocks * (int64_t)block_size > INT_MAX) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return PKV_ERR_SHAPE;
  // the scratch holds the partials of at most kScratchWaves waves
  if (noalloc && max_waves > kScratchWaves) return PKV_ERR_UNSUPPORTED;
  AttnShape s;
  const int rc =
      attn_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, false, &s,
                 noalloc ? kScratchWaves : kMaxWaves);
  if (rc != PKV_OK) return rc;
  // the fused write relies on one query-head chunk per kv head
  if (fused && s.group > 16) return PKV_ERR_UNSUPPORTED;
  // every tile index of the call fits an int32
  if ((int64_t)num_seqs * num_kv_heads * s.group_chunks *
          (((int64_t)max_seq_len + 31) / 32) > INT_MAX)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens)
    return PKV_ERR_NULL;
  if (fused && (!key || !value || !slot_mapping)) return PKV_ERR_NULL;
  if (is_fp8_dtype(cache_dtype) && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (per_token && (!aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return PKV_ERR_ALIGN;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return PKV_ERR_ALIGN;
  if (fused && (!aligned(key, 16) || !aligned(value, 16) ||
                !aligned(slot_mapping, 4)))
    return PKV_ERR_ALIGN;
  if (noalloc) {
    if (s.ws_bytes > kScratchBytes) return PKV_ERR_WORKSPACE;
    const int src = scratch_address(&workspace);
    if (src != PKV_OK) return src;
    workspace_bytes = kScratchBytes;
    if (max_waves == 0) max_waves = kScratchWaves;
  }
  if (!workspace || workspace_bytes < s.ws_bytes) return PKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return PKV_ERR_ALIGN;
  // (debug checks copy and wait, which a call that must stay capturable
  // cannot do: the no-alloc entry skips them)
  if (!noalloc && debug_checks()) {
    std::vector<int32_t> lens, tables, slots;
    int rc = check_tables(block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                          max_seq_len, num_blocks, block_size, stream, &lens,
                          &tables);
    if (rc != PKV_OK) return rc;
    if (fused) {
      if (!fetch_i32(slot_mapping, num_seqs, stream, &slots)) return PKV_ERR_HIP;
      rc = check_slots(slots, num_blocks * (int64_t)block_size);
      if (rc != PKV_OK) return rc;
      // a slot >= 0 is that of the sequence's last position
      for (int32_t q = 0; q < num_seqs; ++q) {
        if (slots[q] < 0) continue;
        const int32_t L = lens[q];
        if (L < 1) return PKV_ERR_RANGE;
        const int64_t phys =
            tables[(size_t)((int64_t)q * max_blocks_per_seq +
                            (L - 1) / block_size)];
        if ((int64_t)slots[q] != phys * block_size + (L - 1) % block_size)
          return PKV_ERR_RANGE;
      }
    }
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
  a.tile_prefix = reinterpret_cast<int32_t*>(ws);
  a.part_m = reinterpret_cast<float*>(ws + s.off_m);
  a.part_l = reinterpret_cast<float*>(ws + s.off_l);
  a.part_o = reinterpret_cast<float*>(ws + s.off_o);
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = s.group;
  a.group_chunks = s.group_chunks;
  a.slot_heads = s.slot_heads;
  a.block_size = block_size;
  a.num_blocks = (int32_t)num_blocks;
  a.max_seq_tokens = max_seq_len;  // within the table's reach (checked)
  a.qk_scale_log2 = scale * 1.4426950408889634f;
  a.scale_per_head = per_head;
  a.scale_per_token = per_token;
  a.kv_stream = kv_stream;
  a.new_key = key;
  a.new_value = value;
  a.slot_mapping = slot_mapping;
  a.num_slots = num_blocks * (int64_t)block_size;
  return launch_attn_decode(a, q_dtype, cache_dtype, head_dim, max_waves,
                            fused, stream) == hipSuccess
             ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" {

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
                      hipStream_t stream) {
  return decode_common(out, query, q_dtype, k_cache, v_cache, cache_dtype,
                       k_scale, v_scale, block_tables, max_blocks_per_seq,
                       seq_lens, max_seq_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, num_blocks, block_size, scale,
                       max_waves, workspace, workspace_bytes, nullptr, nullptr,
                       nullptr, false, stream);
}

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
                              hipStream_t stream) {
  return decode_common(out, query, q_dtype, k_cache, v_cache, cache_dtype,
                       k_scale, v_scale, block_tables, max_blocks_per_seq,
                       seq_lens, max_seq_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, num_blocks, block_size, scale,
                       max_waves, nullptr, 0, nullptr, nullptr, nullptr,
                       false, stream, true);
}

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
                            size_t workspace_bytes, hipStream_t stream) {
  return decode_common(out, query, q_dtype, k_cache, v_cache, cache_dtype,
                       k_scale, v_scale, block_tables, max_blocks_per_seq,
                       seq_lens, max_seq_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, num_blocks, block_size, scale,
                       max_waves, workspace, workspace_bytes, key, value,
                       slot_mapping, true, stream);
}

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
                     size_t workspace_bytes, hipStream_t stream) {
  bool per_head = false, per_token = false, kv_stream = false;
  const int cache_arg = cache_dtype;
  if (!valid_dtype(q_dtype) ||
      !split_cache_dtype(cache_arg, &cache_dtype, &per_head, &per_token,
                         &kv_stream))
    return PKV_ERR_DTYPE;
  if (is_fp8_dtype(q_dtype)) return PKV_ERR_DTYPE;
  if (!is_fp8_dtype(cache_dtype) && q_dtype != cache_dtype) return PKV_ERR_DTYPE;
  if (num_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1 ||
      max_seq_len < 0 || max_waves < 0 || num_query_tokens < 0 ||
      max_query_len < 0 || max_query_len > max_seq_len)
    return PKV_ERR_SHAPE;
  if (num_blocks * (int64_t)block_size > INT_MAX) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return PKV_ERR_SHAPE;
  AttnShape s;
  const int rc =
      attn_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, true, &s);
  if (rc != PKV_OK) return rc;
  const int64_t qbytes = (int64_t)num_query_tokens * num_q_heads * head_dim *
                         dtype_bytes(q_dtype);
  if (qbytes >= ((int64_t)1 << 31)) return PKV_ERR_SHAPE;
  const int32_t tpr = 16 / s.group;
  const int32_t ng =
      multi_groups_per_row(q_dtype, cache_dtype, block_size % 16 == 0,
                           per_token, max_query_len, tpr);
  const int32_t max_rps = (max_query_len + ng * tpr - 1) / (ng * tpr);
  // every unit index of the call, and the merge grid, fit an int32
  const int64_t rows = (int64_t)num_seqs * num_kv_heads * max_rps;
  if (rows > INT_MAX || rows * (((int64_t)max_seq_len + 31) / 32) > INT_MAX)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0)
    return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens ||
      !query_start)
    return PKV_ERR_NULL;
  if (is_fp8_dtype(cache_dtype) && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (per_token && (!aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return PKV_ERR_ALIGN;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) ||
      !aligned(seq_lens, 4) || !aligned(query_start, 4))
    return PKV_ERR_ALIGN;
  if (!workspace || workspace_bytes < s.ws_bytes) return PKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return PKV_ERR_ALIGN;
  if (debug_checks()) {
    std::vector<int32_t> lens, tables, qs;
    const int rc = check_tables(block_tables, max_blocks_per_seq, seq_lens,
                                num_seqs, max_seq_len, num_blocks, block_size,
                                stream, &lens, &tables);
    if (rc != PKV_OK) return rc;
    if (!fetch_i32(query_start, (int64_t)num_seqs + 1, stream, &qs))
      return PKV_ERR_HIP;
    if (qs[0] < 0 || qs[num_seqs] > num_query_tokens) return PKV_ERR_RANGE;
    for (int32_t q = 0; q < num_seqs; ++q) {
      const int64_t n = (int64_t)qs[q + 1] - qs[q];
      if (n < 0 || n > max_query_len || n > lens[q]) return PKV_ERR_RANGE;
    }
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
  a.tile_prefix = reinterpret_cast<int32_t*>(ws);
  a.part_m = reinterpret_cast<float*>(ws + s.off_m);
  a.part_l = reinterpret_cast<float*>(ws + s.off_l);
  a.part_o = reinterpret_cast<float*>(ws + s.off_o);
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = s.group;
  a.group_chunks = 1;
  a.slot_heads = ng * s.slot_heads;  // columns of one partial slot
  a.block_size = block_size;
  a.num_blocks = (int32_t)num_blocks;
  a.max_seq_tokens = max_seq_len;
  a.qk_scale_log2 = scale * 1.4426950408889634f;
  a.scale_per_head = per_head;
  a.scale_per_token = per_token;
  a.kv_stream = kv_stream;
  a.query_start = query_start;
  a.num_query_tokens = num_query_tokens;
  a.max_query_len = max_query_len;
  a.tpr = tpr;
  a.row_tokens = ng * tpr;
  a.max_rps = max_rps;
  a.query_bytes = qbytes;
  return launch_attn_multi(a, q_dtype, cache_dtype, head_dim, max_waves,
                           stream) == hipSuccess
             ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
