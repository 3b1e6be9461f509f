// flk_device.h -- device-side arithmetic shared by the gfx950 codec kernels.
//
// Every helper reproduces one IEEE binary32 step of the codec exactly (the files are built
// with -ffp-contract=off, so no multiply-add is fused unless written as __builtin_fmaf).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flk {

constexpr int kGroup = 64;

// ---- BF16 / FP16 conversions ------------------------------------------------------------

// BF16 is the upper half of a binary32 pattern: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round two binary32 values to BF16 (nearest-even; gfx950 converts in hardware with the
// wave's rounding mode, which is round-to-nearest-even) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Round to BF16 and widen back: the binary32 value of bf16(x).
__device__ __forceinline__ float round_bf16(float x) {
  return __uint_as_float(uint32_t(__builtin_bit_cast(uint16_t, (__bf16)x)) << 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// ---- min / max under the total order -0 < +0 ----------------------------------------------
// IEEE 754-2019 minimum/maximum (v_minimum3_f32 / v_maximum3_f32 on gfx950) order -0
// below +0, so a group's extremes do not depend on the reduction order.
__device__ __forceinline__ float tmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float tmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ---- group parameters -----------------------------------------------------------------------
struct GroupParams {
  float m;        // binary32 value of the FP16 minimum
  float s;        // binary32 value of the FP16 scale (0 for a constant group)
  float rs;       // approximate 1/s (hardware reciprocal, within 1 ulp), unused if s == 0
  uint32_t packed;// FP16 min | FP16 scale << 16
  uint32_t err;   // FLK_DEV_* bits for this group
};

// scale32 = (max - min)/15 with IEEE division, then both rounded to FP16.
__device__ __forceinline__ GroupParams make_params(float mn, float mx) {
  GroupParams p;
  float range = mx - mn;
  float scale32 = range / 15.0f;
  uint16_t m16 = f32_to_f16_bits(mn);
  uint16_t s16 = f32_to_f16_bits(scale32);
  p.packed = uint32_t(m16) | (uint32_t(s16) << 16);
  p.m = f16_bits_to_f32(m16);
  p.s = f16_bits_to_f32(s16);
  p.rs = __builtin_amdgcn_rcpf(p.s);
  uint32_t e = 0;
  // Inf/NaN anywhere in the group make the extremes (or their difference) non-finite.
  if (!(__builtin_isfinite(mn) && __builtin_isfinite(mx))) e |= 1u;
  else if (((m16 & 0x7FFFu) >= 0x7C00u) || ((s16 & 0x7FFFu) >= 0x7C00u)) e |= 2u;
  p.err = e;
  return p;
}

// code = clamp(rint(RN(RN(v - m) / s)), 0, 15) with round-half-even, as a float in 0..15.
// Fast path: q' = RN(y * rs) is within 4 ulp(16) < 2^-18 of RN(y / s) for |q'| < 15, so
// rint(q') equals rint(RN(y / s)) unless q' lies within 2^-15 of a half-integer inside
// (0.5 .. 14.5); only those elements take the correctly rounded division.  Outside
// (0.25, 14.75) both values clamp to the same end code.
__device__ __forceinline__ float code_of(float v, const GroupParams& p) {
  float y = v - p.m;
  float q = y * p.rs;
  float k = __builtin_rintf(q);
  float d = __builtin_fabsf(q - k);
  if (__builtin_expect(d > 0.5f - 0x1p-15f, 0) && q > 0.25f && q < 14.75f) {
    float qe = y / p.s;
    k = __builtin_rintf(qe);
  }
  k = __builtin_amdgcn_fmed3f(k, 0.0f, 15.0f);
  return (p.s == 0.0f) ? 0.0f : k;
}

// decode: min + scale * code in binary32; the product is exact (4-bit code times an 11-bit
// significand), so the fused form rounds once exactly like the separate multiply and add.
__device__ __forceinline__ float decode(float code, float m, float s) { return __builtin_fmaf(code, s, m); }

// Pack 8 codes (floats 0..15) into a uint32, channel 2j in the low nibble of byte j.
__device__ __forceinline__ uint32_t pack_codes8(const float c[8]) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= uint32_t(c[i]) << (4 * i);
  return w;
}

// Nibble i of a packed word as a float.
__device__ __forceinline__ float nib(uint32_t w, int i) { return float((w >> (4 * i)) & 0xFu); }

}  // namespace flk
