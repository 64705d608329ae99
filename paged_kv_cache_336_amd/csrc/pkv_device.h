// pkv_device.h -- element types, gfx950 MFMA steps and fp8 conversions shared
// by the HIP kernels of libpagedkv.  Device-side only; no host API here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) short v4i16_t;

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces addressed by
// lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group, in that
// order.  The address must be 8-byte aligned and point into LDS.
__device__ __forceinline__ v4i16_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(p));
}

__device__ __forceinline__ uint32_t pack_u16x2(short lo, short hi) {
  return (uint32_t)(uint16_t)lo | ((uint32_t)(uint16_t)hi << 16);
}

// Storage element tags (the byte layout of one cache or query element).
struct F32 { typedef float scalar; static constexpr int bytes = 4; };
struct F16 { typedef _Float16 scalar; static constexpr int bytes = 2; };
struct BF16 { typedef __bf16 scalar; static constexpr int bytes = 2; };
struct FP8 { typedef uint8_t scalar; static constexpr int bytes = 1; };    // E4M3
struct FP8E5 { typedef uint8_t scalar; static constexpr int bytes = 1; };  // E5M2

template <typename T> struct is_fp8 { static constexpr bool value = false; };
template <> struct is_fp8<FP8> { static constexpr bool value = true; };
template <> struct is_fp8<FP8E5> { static constexpr bool value = true; };

template <typename A, typename B> struct same { static constexpr bool value = false; };
template <typename A> struct same<A, A> { static constexpr bool value = true; };

// Pointers held in argument structs are generic (flat); reading through a
// global address-space pointer tells the compiler they cannot alias LDS, so a
// wave-uniform read of unmodified memory can become a scalar load.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T*
as_global(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, f);
}

// ---------------------------------------------------------------------------
// One "k32 step" of a 16x16 output tile: acc[m][n] += sum over (group, e) of
// A_lane(m, group)[e] * B_lane(n, group)[e], where lane = row + 16 * group and
// each lane supplies 8 operand elements.  For 16-bit types this is one
// v_mfma_f32_16x16x32_{bf16,f16}; for float32 it is eight 16x16x4 steps, step
// e taking element e of every lane.  Either way A and B pair the same
// (group, element) slots, so callers only need to give matching slots to both
// operands.  Accumulator layout: lane (n + 16 * (m / 4)) holds row m % 4 of
// its 4-float vector.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<BF16> {
  typedef uint32_t operand[4];   // 8 bf16 packed two per register
  __device__ __forceinline__ static f32x4_t step(const operand& a,
                                                 const operand& b, f32x4_t c) {
    u32x4_t av = {a[0], a[1], a[2], a[3]};
    u32x4_t bv = {b[0], b[1], b[2], b[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(av),
                                                   bitcast<bf16x8_t>(bv), c,
                                                   0, 0, 0);
  }
};

template <> struct Mma<F16> {
  typedef uint32_t operand[4];
  __device__ __forceinline__ static f32x4_t step(const operand& a,
                                                 const operand& b, f32x4_t c) {
    u32x4_t av = {a[0], a[1], a[2], a[3]};
    u32x4_t bv = {b[0], b[1], b[2], b[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(av),
                                                  bitcast<f16x8_t>(bv), c,
                                                  0, 0, 0);
  }
};

template <> struct Mma<F32> {
  typedef float operand[8];
  __device__ __forceinline__ static f32x4_t step(const operand& a,
                                                 const operand& b, f32x4_t c) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
};

// ---------------------------------------------------------------------------
// Conversions.  fp8 -> wider types use gfx950's scaled converts with scale 1,
// which decode OCP E4M3 ("fp8") and E5M2 ("bf8") exactly: every value of
// either format is representable in f16, bf16 and f32.  FT selects the
// format (FP8: E4M3, FP8E5: E5M2).
// ---------------------------------------------------------------------------
template <typename FT>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t word, bool hi) {
  f16x2_t v;
  if constexpr (same<FT, FP8E5>::value)
    v = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(word, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(word, 1.0f, false);
  else
    v = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
  return bitcast<uint32_t>(v);
}
template <typename FT>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word, bool hi) {
  bf16x2_t v;
  if constexpr (same<FT, FP8E5>::value)
    v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(word, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(word, 1.0f, false);
  else
    v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true)
           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
  return bitcast<uint32_t>(v);
}
template <typename FT>
__device__ __forceinline__ f32x2_t fp8x2_to_f32x2(uint32_t word, bool hi) {
  if constexpr (same<FT, FP8E5>::value)
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(word, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(word, 1.0f, false);
  else
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, false);
}

// float -> 16-bit storage, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bits(float x, BF16) {
  return bitcast<uint16_t>(static_cast<__bf16>(x));
}
__device__ __forceinline__ uint16_t f32_to_bits(float x, F16) {
  return bitcast<uint16_t>(static_cast<_Float16>(x));
}
__device__ __forceinline__ float bits_to_f32(uint16_t b, BF16) {
  return bitcast<float>(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bits_to_f32(uint16_t b, F16) {
  return static_cast<float>(bitcast<_Float16>(b));
}

// Two floats rounded (to nearest even, as f32_to_bits) into one word, x0 in
// the low half: one packed conversion (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bits(float x0, float x1, BF16) {
  typedef __bf16 v2_t __attribute__((ext_vector_type(2)));
  return bitcast<uint32_t>(__builtin_convertvector(f32x2v_t{x0, x1}, v2_t));
}
__device__ __forceinline__ uint32_t f32x2_to_bits(float x0, float x1, F16) {
  typedef _Float16 v2_t __attribute__((ext_vector_type(2)));
  return bitcast<uint32_t>(__builtin_convertvector(f32x2v_t{x0, x1}, v2_t));
}
// The low / high 16-bit element of a packed word as a float.
__device__ __forceinline__ float lo_bits_to_f32(uint32_t w, BF16) {
  return bitcast<float>(w << 16);
}
__device__ __forceinline__ float hi_bits_to_f32(uint32_t w, BF16) {
  return bitcast<float>(w & 0xFFFF0000u);
}
__device__ __forceinline__ float lo_bits_to_f32(uint32_t w, F16) {
  return static_cast<float>(bitcast<_Float16>(static_cast<uint16_t>(w)));
}
__device__ __forceinline__ float hi_bits_to_f32(uint32_t w, F16) {
  return static_cast<float>(bitcast<_Float16>(static_cast<uint16_t>(w >> 16)));
}

// x minus the low (or high) 16-bit element of the packed word w, in one
// dot2 instruction: the products with -1 and 0 are exact, and so is the
// difference whenever the element is x rounded to the 16-bit type (the
// residual a split into hi + lo parts needs).
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
// (The pair of factors is passed in a scalar register: left to the compiler,
// (-1, 0) becomes the inline constant -1.0, and the residuals came out wrong
// on gfx950.)
template <bool HI>
__device__ __forceinline__ float minus_element(float x, uint32_t w, BF16) {
  uint32_t m = HI ? 0xBF800000u : 0x0000BF80u;  // (0, -1) or (-1, 0)
  asm("" : "+s"(m));
  return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2v_t>(w),
                                         bitcast<bf16x2v_t>(m), x, false);
}
template <bool HI>
__device__ __forceinline__ float minus_element(float x, uint32_t w, F16) {
  uint32_t m = HI ? 0xBC000000u : 0x0000BC00u;
  asm("" : "+s"(m));
  return __builtin_amdgcn_fdot2(bitcast<f16x2v_t>(w), bitcast<f16x2v_t>(m), x,
                                false);
}

// ---------------------------------------------------------------------------
// Wave-wide helpers (wave64).
// ---------------------------------------------------------------------------
// This lane's value and that of lane ^ mask.  Masks 16 and 32 use gfx950's
// row / half swaps (v_permlane16_swap_b32, v_permlane32_swap_b32: VALU
// operations with no LDS round trip); swapping a value with itself leaves
// each lane holding its own value and its partner's, in some order.  Other
// masks go through an LDS permute.
__device__ __forceinline__ void xor_pair(float v, int mask, float& a,
                                         float& b) {
  if (mask == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(
        __float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if (mask == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(
        __float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    a = v;
    b = __shfl_xor(v, mask, 64);
  }
}
__device__ __forceinline__ float xor_max(float v, int mask) {
  float a, b;
  xor_pair(v, mask, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  float a, b;
  xor_pair(v, mask, a, b);
  return a + b;  // (addition commutes exactly: the same sum in both lanes)
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = xor_sum(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = xor_max(v, m);
  return v;
}

// The value of lane n (0..15) of this lane's 16-lane row: a DPP
// row_newbcast move (the control must be a constant; unrolled callers fold
// the switch).
__device__ __forceinline__ float row_broadcast(float v, int n) {
  const int x = __float_as_int(v);
  int r;
#define PKV_ROW_BCAST(k) \
  case k: r = __builtin_amdgcn_update_dpp(0, x, 0x150 + k, 0xF, 0xF, false); break;
  switch (n) {
    PKV_ROW_BCAST(0) PKV_ROW_BCAST(1) PKV_ROW_BCAST(2) PKV_ROW_BCAST(3)
    PKV_ROW_BCAST(4) PKV_ROW_BCAST(5) PKV_ROW_BCAST(6) PKV_ROW_BCAST(7)
    PKV_ROW_BCAST(8) PKV_ROW_BCAST(9) PKV_ROW_BCAST(10) PKV_ROW_BCAST(11)
    PKV_ROW_BCAST(12) PKV_ROW_BCAST(13) PKV_ROW_BCAST(14)
    default: r = __builtin_amdgcn_update_dpp(0, x, 0x15F, 0xF, 0xF, false); break;
  }
#undef PKV_ROW_BCAST
  return __int_as_float(r);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

}  // namespace pkv
