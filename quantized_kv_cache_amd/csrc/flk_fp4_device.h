// flk_fp4_device.h -- decoding of the FP4 streams' scales and element codes, shared by the FP4
// codec kernels and the readers that decode FP4 loops (fused and sparse decode attention).
//
// E2M1 element codes: sign in bit 3, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); a word
// holds 8 codes, byte k the pair (2k, 2k+1), the low nibble the even element.  NVFP4 block
// scales are E4M3 bytes (bias 7, subnormal below 2^-6 in steps of 2^-9, largest finite 448)
// times the stream's binary32 scale; MXFP4 block scales are E8M0 bytes, b = 2^(b - 127).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace flk {

__device__ __forceinline__ float fp4_e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e == 0 ? float(m) * 0x1p-9f : __builtin_ldexpf(1.0f + float(m) * 0.125f, int(e) - 7);
}

// E8M0 byte b -> 2^(b - 127); byte 0 is 2^-127, a binary32 subnormal.
__device__ __forceinline__ float fp4_e8m0_value(uint32_t b) {
  return __uint_as_float(b != 0u ? b << 23 : 0x00400000u);
}

// The 8 codes of a word times a block's binary32 scale bs, RN32(e2m1 * bs), before any BF16
// rounding.  gfx950's v_cvt_scalef32_pk_f32_fp4 with a scale of 1 gives the exact E2M1 values.
typedef float fp4_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp4_decode8(uint32_t cw, float bs, float d[8]) {
  fp4_f32x2 v;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0); d[0] = v.x * bs; d[1] = v.y * bs;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1); d[2] = v.x * bs; d[3] = v.y * bs;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2); d[4] = v.x * bs; d[5] = v.y * bs;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3); d[6] = v.x * bs; d[7] = v.y * bs;
}

// The two E4M3 bytes of 16-bit half HI of w (low byte first) as binary32, by gfx950's
// v_cvt_scalef32_pk_f32_fp8 with a scale of 1: for the non-negative finite bytes a stream's
// block scales use, exactly fp4_e4m3_value of each (checked exhaustively on the GPU).
template <bool HI = false>
__device__ __forceinline__ fp4_f32x2 e4m3x2_value(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
}

// Stream formats of a chain as the readers take them: FMT 0 = INT4 throughout, 1 = INT4 base
// with NVFP4 residual loops, 2 = NVFP4 throughout, 3 = INT4 base with MXFP4 residual loops,
// 4 = MXFP4 throughout.
template <int FMT>
__device__ __forceinline__ constexpr bool loop_nv(int l) { return FMT == 2 || (FMT == 1 && l > 0); }
template <int FMT>
__device__ __forceinline__ constexpr bool loop_mx(int l) { return FMT == 4 || (FMT == 3 && l > 0); }
template <int FMT>
__device__ __forceinline__ constexpr bool loop_fp4(int l) { return loop_nv<FMT>(l) || loop_mx<FMT>(l); }

}  // namespace flk
