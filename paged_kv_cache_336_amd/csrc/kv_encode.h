// kv_encode.h -- encoding of new key/value elements into an fp8 cache (OCP
// E4M3 or E5M2),
// shared by the cache write (cache_ops.hip) and the decode kernel's fused
// write of each sequence's new token (attn_decode.hip).  A stored code is
// e4m3(float32(x) / scale): IEEE float32 division, then the encoder below
// ("How PagedAttention Works in vLLM ...", instagit.com, section
// "write_to_paged_cache": fp8 caches take the value over the per-tensor
// scale).
#ifndef PKV_KV_ENCODE_H
#define PKV_KV_ENCODE_H

#include "pkv_device.h"

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

// OCP E5M2 encoder: round to nearest even on the float32 bit pattern; a
// magnitude that rounds past the largest finite value 57344 (from 61440 on,
// including infinity) becomes infinity (E5M2 keeps IEEE overflow); NaN keeps
// its sign with code S.11111.11.
__device__ __forceinline__ uint32_t encode_e5m2(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t mag = b & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return sign | 0x7Fu;          // NaN
  if (mag < 0x38800000u) {                             // < 2^-14: step 2^-16
    const float q = __uint_as_float(mag) * 65536.0f;   // exact scaling
    return sign | (uint32_t)__builtin_rintf(q);        // 0..4, ties to even
  }
  if (mag >= 0x47700000u) return sign | 0x7Cu;         // >= 61440: infinity
  const uint32_t e = (mag >> 23) - 112u;               // biased for E5M2
  const uint32_t m = (mag >> 21) & 3u;
  const uint32_t rest = mag & 0x1FFFFFu;
  const uint32_t up = (rest > 0x100000u) | ((rest == 0x100000u) & (m & 1u));
  return sign | ((e << 2) + m + up);                   // carry bumps e
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

// Largest magnitude of a 16-element piece (NaN elements ignored).
template <typename ST>
__device__ __forceinline__ float piece_amax(const u32x4_t* in) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(piece_elem<ST>(in, e)));
  return m;
}

// Per-token scale of a row whose largest magnitude is amax: amax over the
// format's largest finite value (IEEE float32 division), 1 for amax 0.
template <typename CT>
__device__ __forceinline__ float row_scale(float amax) {
  const float largest = same<CT, FP8E5>::value ? 57344.f : 448.f;
  return amax == 0.f ? 1.f : amax / largest;
}

// The 16 codes of one 16-element source piece (ST::bytes 16-byte words) in
// the cache's fp8 format CT (FP8: E4M3, FP8E5: E5M2).
template <typename ST, typename CT>
__device__ __forceinline__ u32x4_t encode_piece_fp8(const u32x4_t* in,
                                                    float scale) {
  u32x4_t out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float y = piece_elem<ST>(in, 4 * w + b) / scale;
      const uint32_t code =
          same<CT, FP8E5>::value ? encode_e5m2(y) : encode_e4m3(y);
      word |= code << (8 * b);
    }
    out[w] = word;
  }
  return out;
}

}  // namespace pkv

#endif  // PKV_KV_ENCODE_H
