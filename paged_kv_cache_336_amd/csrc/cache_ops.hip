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
// with 16-byte loads/stores, one grid row per pair.

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// OCP E4M3 ("fn") encoder: round to nearest even on the float32 bit pattern,
// values of magnitude >= 448 (including infinity) saturate to 448, NaN keeps
// its sign with the all-ones code.
__device__ __forceinline__ uint32_t encode_e4m3(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t mag = b & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return sign | 0x7Fu;          // NaN
  if (mag >= 0x43E00000u) return sign | 0x7Eu;         // >= 448
  if (mag < 0x3C800000u) {                             // < 2^-6: step 2^-9
    const float q = __uint_as_float(mag) * 512.0f;     // exact scaling
    return sign | (uint32_t)__builtin_rintf(q);        // 0..8, ties to even
  }
  const uint32_t e = (mag >> 23) - 120u;               // biased for E4M3
  const uint32_t m = (mag >> 20) & 7u;
  const uint32_t rest = mag & 0xFFFFFu;
  const uint32_t up = (rest > 0x80000u) | ((rest == 0x80000u) & (m & 1u));
  uint32_t code = (e << 3) + m + up;                   // carry bumps e
  code = code > 0x7Eu ? 0x7Eu : code;
  return sign | code;
}

// Element e (0..15) of a 16-element source piece held as 16-byte words.
template <typename ST>
__device__ __forceinline__ float piece_elem(const u32x4_t* w, int e);
template <> __device__ __forceinline__ float piece_elem<F32>(const u32x4_t* w, int e) {
  return __uint_as_float(w[e >> 2][e & 3]);
}
template <> __device__ __forceinline__ float piece_elem<F16>(const u32x4_t* w, int e) {
  const uint32_t word = w[e >> 3][(e >> 1) & 3];
  const uint16_t h = (uint16_t)(word >> (16 * (e & 1)));
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
template <> __device__ __forceinline__ float piece_elem<BF16>(const u32x4_t* w, int e) {
  const uint32_t word = w[e >> 3][(e >> 1) & 3];
  return __uint_as_float((word >> (16 * (e & 1))) << 16);
}

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

// fp8 cache: each thread encodes 16 elements into one 16-byte piece.
template <typename ST>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(WriteArgs a) {
  const int pieces = a.row_elems / 16;
  const int64_t total = a.num_tokens * pieces;
  const float ks = *a.k_scale;
  const float vs = *a.v_scale;
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
    if (slot < 0 || slot >= a.num_slots) continue;
    u32x4_t kout, vout;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t kw = 0, vw = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int e = 4 * w + b;
        kw |= encode_e4m3(piece_elem<ST>(kin, e) / ks) << (8 * b);
        vw |= encode_e4m3(piece_elem<ST>(vin, e) / vs) << (8 * b);
      }
      kout[w] = kw;
      vout[w] = vw;
    }
    const int64_t off_dst = (int64_t)slot * a.row_elems + pc * 16;
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

hipError_t launch_cache_write(const WriteArgs& a, int src_dtype,
                              int cache_dtype, hipStream_t stream) {
  if (cache_dtype != PKV_FP8_E4M3) {
    const int ebytes = cache_dtype == PKV_F32 ? 4 : 2;
    const int row_bytes = a.row_elems * ebytes;
    const int grid = grid_for(a.num_tokens * (row_bytes / 16), 256);
    hipLaunchKernelGGL(cache_write_copy_kernel, dim3(grid), dim3(256), 0,
                       stream, a, row_bytes);
  } else {
    const int grid = grid_for(a.num_tokens * (a.row_elems / 16), 256);
    if (src_dtype == PKV_BF16)
      hipLaunchKernelGGL(cache_write_fp8_kernel<BF16>, dim3(grid), dim3(256),
                         0, stream, a);
    else if (src_dtype == PKV_F16)
      hipLaunchKernelGGL(cache_write_fp8_kernel<F16>, dim3(grid), dim3(256),
                         0, stream, a);
    else
      hipLaunchKernelGGL(cache_write_fp8_kernel<F32>, dim3(grid), dim3(256),
                         0, stream, a);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int w = a.prefix ? 3 : 2;
  for (int64_t pair = blockIdx.y; pair < a.num_pairs; pair += gridDim.y) {
    const int64_t src = a.pairs[w * pair];
    const int64_t dst = a.pairs[w * pair + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks)
      continue;  // (a pair outside the pool is the caller's error: skipped)
    int64_t pieces = a.block_bytes / 16;
    if (a.prefix) {  // the first `tokens` token rows, clamped to the block
      const int64_t t = a.pairs[w * pair + 2];
      pieces = (t < 0 ? 0 : (t > a.block_size ? a.block_size : t)) *
               a.token_bytes / 16;
    }
    const uint8_t* ks = static_cast<const uint8_t*>(a.k_cache) + src * a.block_bytes;
    const uint8_t* vs = static_cast<const uint8_t*>(a.v_cache) + src * a.block_bytes;
    uint8_t* kd = static_cast<uint8_t*>(a.k_cache) + dst * a.block_bytes;
    uint8_t* vd = static_cast<uint8_t*>(a.v_cache) + dst * a.block_bytes;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < pieces;
         i += (int64_t)gridDim.x * blockDim.x) {
      const u32x4_t k = *reinterpret_cast<const u32x4_t*>(ks + 16 * i);
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(vs + 16 * i);
      *reinterpret_cast<u32x4_t*>(kd + 16 * i) = k;
      *reinterpret_cast<u32x4_t*>(vd + 16 * i) = v;
    }
  }
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  const int64_t pieces = a.block_bytes / 16;  // the most one copy moves
  int gx = (int)((pieces + 255) / 256);
  if (gx > 64) gx = 64;
  if (gx < 1) gx = 1;
  const unsigned gy = (unsigned)(a.num_pairs < 65535 ? a.num_pairs : 65535);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, gy), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
