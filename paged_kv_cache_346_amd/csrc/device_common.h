// Device-side helpers shared by the gfx950 kernels: vector types, bf16 bit
// manipulation and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// bf16 is carried as raw 16-bit patterns; a 32-bit word holds two of them,
// element 0 in the low half.  Widening to fp32 is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element e of a 16-byte vector, widened to fp32 (bf16: 8 elements; fp32: 4).
template <typename E>
__device__ __forceinline__ float vec_elem(const u32x4& v, int e);
template <>
__device__ __forceinline__ float vec_elem<uint16_t>(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}
template <>
__device__ __forceinline__ float vec_elem<float>(const u32x4& v, int e) {
  return __uint_as_float(v[e]);
}

// Replace element e of a 16-byte vector with the raw value x (a bit copy).
template <typename E>
__device__ __forceinline__ void vec_set(u32x4& v, int e, E x);
template <>
__device__ __forceinline__ void vec_set<uint16_t>(u32x4& v, int e, uint16_t x) {
  const uint32_t w = v[e >> 1];
  v[e >> 1] = (e & 1) ? ((w & 0x0000ffffu) | ((uint32_t)x << 16)) : ((w & 0xffff0000u) | x);
}
template <>
__device__ __forceinline__ void vec_set<float>(u32x4& v, int e, float x) {
  v[e] = __float_as_uint(x);
}
template <>
__device__ __forceinline__ void vec_set<uint8_t>(u32x4& v, int e, uint8_t x) {
  const uint32_t sh = 8 * (e & 3);
  v[e >> 2] = (v[e >> 2] & ~(0xffu << sh)) | ((uint32_t)x << sh);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax with a trailing reference: a column's reference m may trail
// its running maximum by at most kLazyMax (log2 units), so the weights
// exp2(s - m) stay <= 2^8; the accumulator and the weight sum are rescaled
// only when a score passes m + kLazyMax, and out = acc / sum holds for any
// reference.
constexpr float kLazyMax = 8.f;

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}

// Value of `v` held by lane `src` (wave-uniform index), as a scalar.
__device__ __forceinline__ float read_lane(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Within each row of 16 lanes: the value of lane r - 4 (row_shr:4) or r + 4
// (row_shl:4), by DPP; lanes with no such source keep their own value.
__device__ __forceinline__ uint32_t dpp_row_shr4(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t dpp_row_shl4(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x104, 0xf, 0xf, false);
}

// fp8 E4M3 (OCP, gfx950's fp8) to bf16.  Every E4M3 value has at most four
// significant bits and an exponent inside bf16's range, so bf16 holds it
// exactly.  Two codes from one half of a dword (hi selects the upper half),
// first code in the low bf16, in one gfx950 conversion with unit scale.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2_t w) {
  return u32x4{fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
               fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])};
}
// The 16 E4M3 codes of a 16-byte vector as fp32 values (exact), code e in f[e].
__device__ __forceinline__ void fp8x16_to_f32(const u32x4& w, float (&f)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    f[4 * i] = lo[0];
    f[4 * i + 1] = lo[1];
    f[4 * i + 2] = hi[0];
    f[4 * i + 3] = hi[1];
  }
}
__device__ __forceinline__ u32x2_t fp8x4_to_bf16(uint32_t w) {
  return u32x2_t{fp8x2_to_bf16x2<false>(w), fp8x2_to_bf16x2<true>(w)};
}

// fp32 to fp8 E4M3 code: nearest value, ties to an even mantissa, magnitudes
// at or above 448 (the largest finite value) saturate to 448, NaN gives 0x7F.
// Written from the format: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
// exponent field 0 holds m * 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                      // NaN
  const float af = __uint_as_float(a);
  if (af >= 448.f) return sign | 0x7eu;
  if (af < 0.015625f) {                                   // below 2^-6: steps of 2^-9
    const uint32_t q = (uint32_t)__builtin_rintf(af * 512.f);  // exact scaling; 8 = 2^-6
    return sign | q;
  }
  // keep 3 of the 23 mantissa bits, rounding the 20 dropped ones to nearest even;
  // a carry moves into the exponent field
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  const int e = (int)(r >> 23) - 127;                     // -6 .. 8
  return sign | ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);
}

}  // namespace pkv
