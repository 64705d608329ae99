// cache_ops.hip -- slot-mapped cache write and copy-on-write block copy.
//
// cache_write ("How PagedAttention Works in vLLM ...", instagit.com, section
// "write_to_paged_cache: Direct In-Place Updates"): new key/value rows
// [T, kv_heads, head_dim] are scattered in place to slot_mapping[t] =
// block * block_size + offset of pools [num_blocks, block_size, kv_heads,
// head_dim]; no staging buffer.  One thread per 16-byte piece of destination
// row, so every store is a full 16-byte vector store and a token's row is
// written by consecutive threads.
//
// copy_blocks ("PagedAttention", shubhamtatvamasi.com, section "Sharing and
// copy-on-write"): each (src, dst) pair copies a whole block of both pools
// with 16-byte loads/stores, one grid row per pair -- and, for the pools of
// every layer at once (a block is "16 tokens x all layers' K and V", the
// same page's table), one grid slice per layer.

#include "kv_encode.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// Same dtype: bit copy of 16-byte pieces.
__global__ __launch_bounds__(256) void cache_write_copy_kernel(WriteArgs a,
                                                               int row_bytes) {
  const int pieces = row_bytes / 16;
  const int64_t total = a.num_tokens * pieces;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / pieces;
    const int pc = (int)(i - t * pieces);
    const int32_t slot = a.slot_mapping[t];
    if (slot < 0 || slot >= a.num_slots) continue;
    const int64_t off_src = t * row_bytes + pc * 16;
    const int64_t off_dst = (int64_t)slot * row_bytes + pc * 16;
    const u32x4_t k = *reinterpret_cast<const u32x4_t*>(
        static_cast<const uint8_t*>(a.key) + off_src);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
        static_cast<const uint8_t*>(a.value) + off_src);
    *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.k_cache) + off_dst) = k;
    *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.v_cache) + off_dst) = v;
  }
}

// fp8 cache (CT: E4M3 or E5M2): each thread encodes 16 elements into one
// 16-byte piece; with per-head scales, piece pc belongs to kv head
// 16 pc / head_dim.  PT (per-token scales): the head_dim / 16 consecutive
// threads holding one (token, kv head) row -- aligned groups of a wave,
// since the pieces of a token start at a multiple of the group size and the
// grid stride is a multiple of 64 -- take the row's largest magnitude over
// xor shuffles, and the row's scale is that over the format's largest
// finite value (1 for a row without a nonzero element); the group's first
// thread stores it beside the row.
template <typename ST, typename CT, bool PT>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(WriteArgs a) {
  const int pieces = a.row_elems / 16;
  const int64_t total = a.num_tokens * pieces;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / pieces;
    const int pc = (int)(i - t * pieces);
    // the slot, the scales and the source piece are requested together
    const int32_t slot = a.slot_mapping[t];
    constexpr int NW = ST::bytes;  // 16-byte words per 16-element piece
    const int64_t e0 = t * a.row_elems + pc * 16;
    const u32x4_t* ksrc = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint8_t*>(a.key) + e0 * ST::bytes);
    const u32x4_t* vsrc = reinterpret_cast<const u32x4_t*>(
        static_cast<const uint8_t*>(a.value) + e0 * ST::bytes);
    u32x4_t kin[NW], vin[NW];
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      kin[q] = ksrc[q];
      vin[q] = vsrc[q];
    }
    float ksc, vsc;
    const int64_t off_dst = (int64_t)slot * a.row_elems + pc * 16;
    if constexpr (PT) {
      // every thread of the group takes part (same token, same slot)
      float km = piece_amax<ST>(kin), vm = piece_amax<ST>(vin);
      for (int o = 1; o < a.head_dim / 16; o <<= 1) {
        km = fmaxf(km, __shfl_xor(km, o, 64));
        vm = fmaxf(vm, __shfl_xor(vm, o, 64));
      }
      ksc = row_scale<CT>(km);
      vsc = row_scale<CT>(vm);
      if (slot < 0 || slot >= a.num_slots) continue;
      if (pc % (a.head_dim / 16) == 0) {
        const int64_t at = off_dst / a.head_dim;  // slot * hkv + head
        a.k_token_scales[at] = ksc;
        a.v_token_scales[at] = vsc;
      }
    } else {
      if (slot < 0 || slot >= a.num_slots) continue;
      const int h = a.scale_per_head ? pc * 16 / a.head_dim : 0;
      ksc = a.k_scale[h];
      vsc = a.v_scale[h];
    }
    const u32x4_t kout = encode_piece_fp8<ST, CT>(kin, ksc);
    const u32x4_t vout = encode_piece_fp8<ST, CT>(vin, vsc);
    *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.k_cache) + off_dst) = kout;
    *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.v_cache) + off_dst) = vout;
  }
}

static int grid_for(int64_t work, int threads) {
  int64_t g = (work + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

template <typename CT, bool PT>
static void launch_fp8(const WriteArgs& a, int src_dtype, hipStream_t stream) {
  const int grid = grid_for(a.num_tokens * (a.row_elems / 16), 256);
  if (src_dtype == PKV_BF16)
    hipLaunchKernelGGL((cache_write_fp8_kernel<BF16, CT, PT>), dim3(grid),
                       dim3(256), 0, stream, a);
  else if (src_dtype == PKV_F16)
    hipLaunchKernelGGL((cache_write_fp8_kernel<F16, CT, PT>), dim3(grid),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((cache_write_fp8_kernel<F32, CT, PT>), dim3(grid),
                       dim3(256), 0, stream, a);
}

hipError_t launch_cache_write(const WriteArgs& a, int src_dtype,
                              int cache_dtype, hipStream_t stream) {
  if (cache_dtype != PKV_FP8_E4M3 && cache_dtype != PKV_FP8_E5M2) {
    const int ebytes = cache_dtype == PKV_F32 ? 4 : 2;
    const int row_bytes = a.row_elems * ebytes;
    const int grid = grid_for(a.num_tokens * (row_bytes / 16), 256);
    hipLaunchKernelGGL(cache_write_copy_kernel, dim3(grid), dim3(256), 0,
                       stream, a, row_bytes);
  } else if (cache_dtype == PKV_FP8_E4M3) {
    if (a.k_token_scales) launch_fp8<FP8, true>(a, src_dtype, stream);
    else launch_fp8<FP8, false>(a, src_dtype, stream);
  } else {
    if (a.k_token_scales) launch_fp8<FP8E5, true>(a, src_dtype, stream);
    else launch_fp8<FP8E5, false>(a, src_dtype, stream);
  }
  return hipGetLastError();
}

// P: the unit each thread moves, a 16-byte vector (pools) or one float
// (per-token scale arrays, whose blocks need not be multiples of 16 bytes).
template <typename P>
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int w = a.prefix ? 3 : 2;
  // grid z: the layer whose pools this workgroup copies in (one block id
  // names the same block in every layer's pools)
  const int64_t lofs = (int64_t)blockIdx.z * a.layer_stride;
  for (int64_t pair = blockIdx.y; pair < a.num_pairs; pair += gridDim.y) {
    const int64_t src = a.pairs[w * pair];
    const int64_t dst = a.pairs[w * pair + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks)
      continue;  // (a pair outside the pool is the caller's error: skipped)
    int64_t pieces = a.block_bytes / (int64_t)sizeof(P);
    if (a.prefix) {  // the first `tokens` token rows, clamped to the block
      const int64_t t = a.pairs[w * pair + 2];
      pieces = (t < 0 ? 0 : (t > a.block_size ? a.block_size : t)) *
               a.token_bytes / (int64_t)sizeof(P);
    }
    uint8_t* kl = static_cast<uint8_t*>(a.k_cache) + lofs;
    uint8_t* vl = static_cast<uint8_t*>(a.v_cache) + lofs;
    const uint8_t* ks = kl + src * a.block_bytes;
    const uint8_t* vs = vl + src * a.block_bytes;
    uint8_t* kd = kl + dst * a.block_bytes;
    uint8_t* vd = vl + dst * a.block_bytes;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < pieces;
         i += (int64_t)gridDim.x * blockDim.x) {
      const P k = reinterpret_cast<const P*>(ks)[i];
      const P v = reinterpret_cast<const P*>(vs)[i];
      reinterpret_cast<P*>(kd)[i] = k;
      reinterpret_cast<P*>(vd)[i] = v;
    }
  }
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  const int64_t pieces = a.block_bytes / a.piece_bytes;  // most per copy
  int gx = (int)((pieces + 255) / 256);
  if (gx > 64) gx = 64;
  if (gx < 1) gx = 1;
  const unsigned gy = (unsigned)(a.num_pairs < 65535 ? a.num_pairs : 65535);
  if (a.piece_bytes == 4)
    hipLaunchKernelGGL(copy_blocks_kernel<uint32_t>,
                       dim3(gx, gy, a.num_layers), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<u32x4_t>,
                       dim3(gx, gy, a.num_layers), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
