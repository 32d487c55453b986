// Device-side helpers for the gfx950 kernels: vector types, bfloat16
// conversion, cross-lane reductions and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats -> packed bfloat16 pair (lo in bits 0..15), round to nearest
// even; one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_t{lo, hi}, bf16x2_t));
}

// Byte-select of two dwords (v_perm_b32): result byte i = selector byte i
// indexes the 8 bytes {lo word b (bytes 0..3), hi word a (bytes 4..7)}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(a, b, sel);
}
// {lo16(x), lo16(y)} and {hi16(x), hi16(y)} packed into one dword.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) { return perm_b32(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) { return perm_b32(y, x, 0x07060302u); }

template <typename T>
__device__ __forceinline__ T bitcast(const void* p) {
  T v;
  __builtin_memcpy(&v, p, sizeof(T));
  return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x4 as_bf16x4(u32x2 v) { return __builtin_bit_cast(bf16x4, v); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// max(x, x of lane ^ 32) with one v_permlane32_swap (no LDS round trip).
__device__ __forceinline__ float max_lane_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// acc + lo + hi of a packed bfloat16 pair (v_dot2_f32_bf16 against {1, 1}).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w), __builtin_bit_cast(bf16x2v, 0x3f803f80u), acc,
                                         false);
}

__device__ __forceinline__ floatx4 mfma_16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_16x16x16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma_32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j receives component j%4 of the four 16-bit values addressed by each
// of the lanes 4t + j/4 (t = 0..3), in t order.
typedef short shortx4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) shortx4_t lds_shortx4;
  const shortx4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// Global loads; 16 / 8 / 4 byte vectors.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }

// FP8 (OCP E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinity, S.1111.111 = NaN, largest finite 448).
//
// Decode: bytes 0-1 (HI = false) or 2-3 (HI = true) of w to a bf16 pair, with
// gfx950's v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact: every E4M3 value is
// a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Four FP8 values of a dword (byte order = element order) to four bf16.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  return u32x2{fp8x2_to_bf16x2<false>(w), fp8x2_to_bf16x2<true>(w)};
}
// Eight FP8 values (two dwords) to eight bf16.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 w) {
  return as_bf16x8(u32x4{fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x), fp8x2_to_bf16x2<false>(w.y),
                         fp8x2_to_bf16x2<true>(w.y)});
}
// Encode: nearest E4M3 value, ties to the even mantissa; magnitudes of 448
// and beyond (infinity included) saturate to 448; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return s | 0x7fu;       // NaN
  if (a >= 0x43e00000u) return s | 0x7eu;      // >= 448
  if (a < 0x3c800000u) {                        // below 2^-6: multiples of 2^-9
    return s | uint32_t(__builtin_rintf(__uint_as_float(a) * 512.f));  // 0..8; 8 is 2^-6
  }
  const uint32_t m = a & 0x7fffffu;
  uint32_t e = (a >> 23) - 120u;                // exponent re-biased from 127 to 7: 1..15
  uint32_t r = (m + 0x7ffffu + ((m >> 20) & 1u)) >> 20;
  if (r == 8u) {
    r = 0u;
    ++e;
  }
  return s | (e << 3) | r;                      // below 448: never reaches e = 15 with r = 7
}

}  // namespace rtk
