// w6_device.h -- gfx950 device helpers shared by the W6Ax kernels.
//
// Weight unit (16 six-bit codes in 3 dwords, 4-bit plane + 2-bit plane as in the
// ZeroQuant(4+2) split) -> four int8x4 MFMA operand dwords whose bytes are 4*q:
// the 6-bit field lands in bits 2..7 of each byte and bits 0..1 are zero, so the
// sign comes for free and an int8 MFMA over these bytes yields exactly 4 * (the
// group dot of the FlexQ BTC section).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace flexq {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;          // K-group of the method (BTC section: 128-deep K groups)
constexpr int kUnitsPerGroup = 8;    // 16 codes per unit
constexpr int kUnitDwords = 3;

// MFMA accumulator start for the fused rescale: the float 1.5 * 2^23.  A group's
// int32 products started from these bits end as the bits of the float
// F = 12582912 + 4d exactly while |4d| < 2^22 (always: |d| <= 128 * 32 * 127), and
// fma(F, s / 4, -12582912 * s / 4) is then the single rounding of d * s for any
// scale s with at most 22 significant bits (fp16 scales have 11).
constexpr uint32_t kMagic = 0x4B400000u;
constexpr float kMagicF = 12582912.0f;

// Decode one unit into 16 int8 lanes holding 4*q, code i in byte i.
__device__ __forceinline__ i32x4 unpack_unit_x4(uint32_t d0, uint32_t d1, uint32_t d2) {
  i32x4 e;
  e[0] = (int32_t)(((d0 << 2) & 0x3C3C3C3Cu) | ((d2 << 6) & 0xC0C0C0C0u));
  e[1] = (int32_t)(((d0 >> 2) & 0x3C3C3C3Cu) | ((d2 << 4) & 0xC0C0C0C0u));
  e[2] = (int32_t)(((d1 << 2) & 0x3C3C3C3Cu) | ((d2 << 2) & 0xC0C0C0C0u));
  e[3] = (int32_t)(((d1 >> 2) & 0x3C3C3C3Cu) | (d2 & 0xC0C0C0C0u));
  return e;
}

// Encode 16 codes (q in [-32, 31]) into one unit.
__device__ __forceinline__ u32x3 pack_unit(const int q[16]) {
  uint32_t d0 = 0, d1 = 0, d2 = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t v0 = (uint32_t)q[j] & 63u, v1 = (uint32_t)q[4 + j] & 63u;
    uint32_t v2 = (uint32_t)q[8 + j] & 63u, v3 = (uint32_t)q[12 + j] & 63u;
    d0 |= ((v0 & 15u) | ((v1 & 15u) << 4)) << (8 * j);
    d1 |= ((v2 & 15u) | ((v3 & 15u) << 4)) << (8 * j);
    d2 |= ((v0 >> 4) | ((v1 >> 4) << 2) | ((v2 >> 4) << 4) | ((v3 >> 4) << 6)) << (8 * j);
  }
  u32x3 r;
  r[0] = d0;
  r[1] = d1;
  r[2] = d2;
  return r;
}

// The same unit from 16 int8 codes (each in [-32, 31]) held four per dword: bytes of
// c0 = codes 0-3, c1 = 4-7, c2 = 8-11, c3 = 12-15.  The low nibble of each byte is
// the code's 4-bit part and bits 4-5 its 2-bit part, so the planes come out with
// masks and shifts on whole dwords.
__device__ __forceinline__ u32x3 pack_codes16(uint32_t c0, uint32_t c1, uint32_t c2,
                                              uint32_t c3) {
  u32x3 r;
  r[0] = (c0 & 0x0F0F0F0Fu) | ((c1 & 0x0F0F0F0Fu) << 4);
  r[1] = (c2 & 0x0F0F0F0Fu) | ((c3 & 0x0F0F0F0Fu) << 4);
  r[2] = ((c0 >> 4) & 0x03030303u) | (((c1 >> 4) & 0x03030303u) << 2) |
         (((c2 >> 4) & 0x03030303u) << 4) | (((c3 >> 4) & 0x03030303u) << 6);
  return r;
}

// First dword of unit (n, u = k/16) of an N x K packed weight.
__host__ __device__ __forceinline__ int64_t unit_dword(int64_t n, int64_t u, int64_t K) {
  return 3 * (((n >> 4) * (K >> 4) + u) * 16 + (n & 15));
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// binary32 -> binary16, round to nearest even, of an already rounded binary32 value.
// The empty asm hides where `f` came from: hipcc 7.2 otherwise folds a final
// fmaf + conversion into one v_fma_mix (a single rounding straight to fp16), which
// differs from rounding to fp32 first whenever the fp32 result is an fp16 tie.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  asm volatile("" : "+v"(f));
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32
}

// max over the 16 lanes of a DPP row (butterfly: swap pairs, swap pairs of pairs,
// mirror within 8 lanes, mirror within 16 lanes)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
  return x;
}

// Code of one activation: rint(RN(v / s)) clamped to +-qmax, s > 0.  The quotient
// is first taken as q = RN(v * r) with r = RN(1 / s); |v / s| <= 128, so q is within
// 2^-16 of v / s, and the correctly rounded quotient within 2^-17 of it.  When q
// is at least 2^-15 away from the nearest odd multiple of 1/2 (the rounding
// boundaries), both round to the same integer; otherwise (a few activations in ten
// thousand on typical inputs) the exact quotient is formed.  Every step of the test is exact: q - rint(q)
// and its distance to 1/2 are differences of nearby fp32 values.
__device__ __forceinline__ int quant_code(float v, float s, float r, int qmax) {
  const float q = v * r;
  float k = rintf(q);
  if (fabsf(fabsf(q - k) - 0.5f) < 0x1p-15f) k = rintf(v / s);
  const int c = (int)k;
  return c > qmax ? qmax : (c < -qmax ? -qmax : c);
}

// Activation group quantization, one lane's share: 8 consecutive fp16 activations
// of a 128-deep group whose other 120 sit in the other 15 lanes of this lane's DPP
// row.  Returns the 8 int8 codes (byte i = code i) and sets s to the group's scale
// amax / qmax (+0 for an all-zero group, whose codes are 0).  Every lane of the
// wave must take part (the group max is a DPP butterfly).
__device__ __forceinline__ u32x2 quant8_row16(const u32x4 h, int qmax, float& s) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = half_bits_to_float((uint16_t)(h[i] & 0xFFFFu));
    v[2 * i + 1] = half_bits_to_float((uint16_t)(h[i] >> 16));
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = row16_max(amax);
  s = amax / (float)qmax;
  const float r = 1.0f / s;
  u32x2 out = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = s != 0.0f ? quant_code(v[i], s, r, qmax) : 0;
    out[i >> 2] |= (uint32_t)(c & 0xFF) << (8 * (i & 3));
  }
  return out;
}

// 16x16x64 int8 MFMA: lane l supplies A row (l % 16) and B column (l % 16), 16 bytes
// each, for k-block (l / 16); D lane l holds column l % 16, rows 4*(l/16) .. +3.
__device__ __forceinline__ i32x4 mfma16(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 32x32x32 int8 MFMA: lane l supplies A row (l % 32) and B column (l % 32), 16 bytes
// each, for k-block (l / 32); D lane l holds column l % 32 and, in register r,
// row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ i32x16 mfma32(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// f(integral_constant<int, K>) for K = 0 .. n-1, in order (compile-time indices in
// unrolled loops).
template <class F, int... K>
__device__ __forceinline__ void unroll(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}

}  // namespace flexq
