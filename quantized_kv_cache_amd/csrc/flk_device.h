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

// Round to BF16 and widen back: the binary32 value of bf16(x), in one instruction
// (v_cvt_pk_bf16_f32 with a zero low half writes bf16(x) << 16, which is that value).
__device__ __forceinline__ float round_bf16(float x) {
  return __uint_as_float(pack_bf16x2(0.0f, x));
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

// RN(x / 15), the IEEE quotient, for every binary32 x other than -0 (a range is never -0):
// q0 = RN(x * RN(1/15)) is within an ulp of x / 15, the remainder x - 15 q0 is exact in an
// fma, and one fma step from it rounds correctly.  Three instructions where the division
// takes about ten; checked against the IEEE division for every finite binary32 x >= +0
// (tests/native/hw_arith_check.hip).  An infinite x gives NaN instead of Inf (an error
// group either way).
__device__ __forceinline__ float div15(float x) {
  constexpr float r = 0x1.111112p-4f;   // RN(1/15)
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, 15.0f, x);
  return __builtin_fmaf(e, r, q0);
}

// scale32 = (max - min)/15 with IEEE division, then both rounded to FP16.
__device__ __forceinline__ GroupParams make_params(float mn, float mx) {
  GroupParams p;
  float range = mx - mn;
  float scale32 = div15(range);
  // the FP16 scale is the FP16 rounding of the binary32 quotient: without this barrier the
  // compiler folds the conversion into the last fma (v_fma_mixlo_f16), which rounds the exact
  // value to FP16 once and differs where the quotient is an FP16 midpoint
  asm volatile("" : "+v"(scale32));
  uint16_t m16 = f32_to_f16_bits(mn);
  uint16_t s16 = f32_to_f16_bits(scale32);
  p.packed = uint32_t(m16) | (uint32_t(s16) << 16);
  p.m = f16_bits_to_f32(m16);
  p.s = f16_bits_to_f32(s16);
  p.rs = p.s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(p.s);   // constant group: every q is 0
  // Inf/NaN anywhere in the group make the minimum or the scale Inf/NaN in FP16, and so does
  // an FP16 overflow: an all-ones exponent in either half of the packed params (adding 1 to
  // the exponent field carries into the half's sign bit exactly then) flags the group, which
  // then tells the two cases apart.
  p.err = 0;
  const uint32_t ex = p.packed & 0x7C007C00u;
  if (__builtin_expect(((ex + 0x04000400u) & 0x80008000u) != 0u, 0))
    p.err = (__builtin_isfinite(mn) && __builtin_isfinite(mx)) ? 2u : 1u;
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

// Codes of n values against one group's params, as floats 0..15.  The fast path rounds
// q' = RN(y * rs) clamped to [0, 15]; it can differ from the exact rule only where q' lies
// within 2^-15 of a half-integer (see code_of), and one test over all n values sends the
// lane to the correctly rounded division in that case.  Clamping before rounding equals
// rounding before clamping, and a clamped value (0 or 15) is never near a half-integer.
template <int N>
__device__ __forceinline__ void codes_of(const float v[N], const GroupParams& p, float k[N]) {
  float y[N], dev = 0.0f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    y[e] = v[e] - p.m;
    const float qc = __builtin_amdgcn_fmed3f(y[e] * p.rs, 0.0f, 15.0f);
    k[e] = __builtin_rintf(qc);
    dev = __builtin_fmaxf(dev, __builtin_fabsf(qc - k[e]));
  }
  if (__builtin_expect(dev > 0.5f - 0x1p-15f, 0)) {
#pragma unroll
    for (int e = 0; e < N; ++e) k[e] = __builtin_rintf(__builtin_amdgcn_fmed3f(y[e] / p.s, 0.0f, 15.0f));
  }
}

// Codes of n values, each against its own group's params (K: a group per channel), with the
// fast path and the single fallback test of codes_of.  A group of scale 0 (its reciprocal is 0,
// so the fast path gives code 0) keeps code 0 in the fallback too.
template <int N>
__device__ __forceinline__ void codes_of_each(const float v[N], const GroupParams (&p)[N], float k[N]) {
  float y[N], dev = 0.0f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    y[e] = v[e] - p[e].m;
    const float qc = __builtin_amdgcn_fmed3f(y[e] * p[e].rs, 0.0f, 15.0f);
    k[e] = __builtin_rintf(qc);
    dev = __builtin_fmaxf(dev, __builtin_fabsf(qc - k[e]));
  }
  if (__builtin_expect(dev > 0.5f - 0x1p-15f, 0)) {
#pragma unroll
    for (int e = 0; e < N; ++e)
      k[e] = p[e].s == 0.0f ? 0.0f : __builtin_rintf(__builtin_amdgcn_fmed3f(y[e] / p[e].s, 0.0f, 15.0f));
  }
}

// decode: min + scale * code in binary32; the product is exact (4-bit code times an 11-bit
// significand), so the fused form rounds once exactly like the separate multiply and add.
__device__ __forceinline__ float decode(float code, float m, float s) { return __builtin_fmaf(code, s, m); }

// Pack 8 codes (floats 0..15, exact integers) into a uint32 with v_cvt_pk_u8_f32: the even
// channels fill the bytes of one word, the odd channels another, shifted into the high
// nibbles.
__device__ __forceinline__ uint32_t pack_codes8_u8(const float c[8]) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_u8_f32(c[0], 0, lo);
  lo = __builtin_amdgcn_cvt_pk_u8_f32(c[2], 1, lo);
  lo = __builtin_amdgcn_cvt_pk_u8_f32(c[4], 2, lo);
  lo = __builtin_amdgcn_cvt_pk_u8_f32(c[6], 3, lo);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(c[1], 0, hi);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(c[3], 1, hi);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(c[5], 2, hi);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(c[7], 3, hi);
  return lo | (hi << 4);
}

// Pack 8 codes (floats 0..15) into a uint32, channel 2j in the low nibble of byte j.
__device__ __forceinline__ uint32_t pack_codes8(const float c[8]) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= uint32_t(c[i]) << (4 * i);
  return w;
}

// Nibble i of a packed word as a float.
__device__ __forceinline__ float nib(uint32_t w, int i) { return float((w >> (4 * i)) & 0xFu); }

// Keeps a value in a register as computed (an empty asm barrier), so the byte-wise
// conversion below is not re-folded into per-nibble shifts and masks.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The 8 codes of a packed word as floats in channel order: even channels from the low
// nibbles, odd from the high nibbles, each byte converted with v_cvt_f32_ubyteN.
__device__ __forceinline__ void codes8_to_f32(uint32_t cw, float c[8]) {
  const uint32_t lo = opaque(cw & 0x0F0F0F0Fu);
  const uint32_t hi = opaque((cw >> 4) & 0x0F0F0F0Fu);
  c[0] = float(lo & 0xFFu);
  c[2] = float((lo >> 8) & 0xFFu);
  c[4] = float((lo >> 16) & 0xFFu);
  c[6] = float(lo >> 24);
  c[1] = float(hi & 0xFFu);
  c[3] = float((hi >> 8) & 0xFFu);
  c[5] = float((hi >> 16) & 0xFFu);
  c[7] = float(hi >> 24);
}

// Round 8 binary32 values to BF16 in place, one instruction each; x[] then holds the
// binary32 values of the rounded numbers.
__device__ __forceinline__ void round_bf16x8_inplace(float x[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = round_bf16(x[e]);
}

// Pack 8 binary32 values that are already exactly BF16 (low halves zero): the high halves.
__device__ __forceinline__ uint4 pack_exact_bf16x8(const float x[8]) {
  uint4 w;
  w.x = __builtin_amdgcn_perm(__float_as_uint(x[1]), __float_as_uint(x[0]), 0x07060302u);
  w.y = __builtin_amdgcn_perm(__float_as_uint(x[3]), __float_as_uint(x[2]), 0x07060302u);
  w.z = __builtin_amdgcn_perm(__float_as_uint(x[5]), __float_as_uint(x[4]), 0x07060302u);
  w.w = __builtin_amdgcn_perm(__float_as_uint(x[7]), __float_as_uint(x[6]), 0x07060302u);
  return w;
}

// Round 8 binary32 values to BF16 in place (pairs through v_cvt_pk_bf16_f32) and return
// them packed; x[] then holds the binary32 values of the rounded numbers.
__device__ __forceinline__ uint4 round_bf16x8(float x[8]) {
  uint4 w;
  w.x = pack_bf16x2(x[0], x[1]);
  w.y = pack_bf16x2(x[2], x[3]);
  w.z = pack_bf16x2(x[4], x[5]);
  w.w = pack_bf16x2(x[6], x[7]);
  x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xFFFF0000u);
  x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xFFFF0000u);
  x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xFFFF0000u);
  x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xFFFF0000u);
  return w;
}

// acc[e] = bf16(acc[e]) + bf16(d[e]) in binary32, for 8 elements: v_cvt_pk_bf16_f32 rounds
// the two operands into the halves of one word, and v_dot2_f32_bf16 against (1, 1) with a zero
// addend sums them -- two instructions per element instead of three.  The dot's binary32 sum
// is not always the correctly rounded one when the exponents are 16 or more apart, but every
// such sum lies far from a BF16 rounding boundary, and each sum of the chain is rounded to
// BF16 before it is used, so the BF16 results equal those of v_add_f32 (checked on the GPU
// for every pair of +0 / finite normal BF16 values).  The eight dots sit in one asm statement
// followed by the 3 wait states a VALU read of a dot's result needs; the compiler does not
// know the instructions inside an asm statement and inserts no wait states for them.
__device__ __forceinline__ void add_rounded_bf16x8(float acc[8], const float d[8], uint32_t ones) {
  uint32_t p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = pack_bf16x2(acc[e], d[e]);
  asm("v_dot2_f32_bf16 %0, %8, %16, 0\n\t"
      "v_dot2_f32_bf16 %1, %9, %16, 0\n\t"
      "v_dot2_f32_bf16 %2, %10, %16, 0\n\t"
      "v_dot2_f32_bf16 %3, %11, %16, 0\n\t"
      "v_dot2_f32_bf16 %4, %12, %16, 0\n\t"
      "v_dot2_f32_bf16 %5, %13, %16, 0\n\t"
      "v_dot2_f32_bf16 %6, %14, %16, 0\n\t"
      "v_dot2_f32_bf16 %7, %15, %16, 0\n\t"
      "s_nop 2"
      : "=&v"(acc[0]), "=&v"(acc[1]), "=&v"(acc[2]), "=&v"(acc[3]), "=&v"(acc[4]), "=&v"(acc[5]),
        "=&v"(acc[6]), "=&v"(acc[7])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]), "s"(ones));
}
// BF16 1.0 in both halves, in a scalar register (the three-operand dot2 takes no literal)
__device__ __forceinline__ uint32_t bf16_ones() {
  uint32_t x;
  asm volatile("s_mov_b32 %0, 0x3f803f80" : "=s"(x));
  return x;
}

// binary16 bits of the low / high half of a word -> binary32 (exact; a 4-bit code as the bit
// pattern gives the subnormal code * 2^-24)
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// The 8 codes of a code word (code e in bits 4e .. 4e+3) as binary16 subnormals: word q holds
// code q in its low half and code q + 4 in its high half.
__device__ __forceinline__ void codes8_to_f16_halves(uint32_t cw, uint32_t wq[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) wq[q] = (cw >> (4 * q)) & 0x000F000Fu;
}

constexpr float kCodeScale = 16777216.0f;   // 2^24: scale * 2^24 times code * 2^-24 is code * scale

// ---- buffer-resource accesses ----------------------------------------------------------------
// A raw buffer resource holds a scalar base address and a byte range; an access adds a
// 32-bit per-lane offset (VGPR) and a 32-bit wave-uniform offset (SGPR), so per-row
// addressing costs no vector instructions.  Lane offsets at or past the range read zero and
// drop stores.  kBufDword3 is the gfx9-family descriptor word for raw 32-bit access.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kBufDword3 = 0x00020000;
constexpr int kCacheStream = 2;     // nontemporal: stream past the caches

// The row offset must be wave-uniform; readfirstlane states it so the compiler never builds
// a per-lane loop around an access (it is free when the value already is a scalar).
__device__ __forceinline__ int soffset(uint32_t soff) { return __builtin_amdgcn_readfirstlane(int(soff)); }

__device__ __forceinline__ BufRsrc make_buf(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), kBufDword3);
}
template <int AUX = 0>
__device__ __forceinline__ uint32_t buf_ld32(BufRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), soffset(soff), AUX);
}
template <int AUX = 0>
__device__ __forceinline__ uint4 buf_ld128(BufRsrc r, uint32_t voff, uint32_t soff) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  const v4 v = __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), soffset(soff), AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_st32(uint32_t w, BufRsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(w, r, int(voff), soffset(soff), AUX);
}
// A store of more than 64 bits reads its data VGPRs after it issues, so a VALU write of them
// needs a wait state in between.  The compiler inserts it only for a store whose scalar offset
// is not a register; on gfx950 a store with an SGPR offset showed the same hazard (the last
// four lanes of each 16-lane row stored the overwritten value of data dwords whose registers
// the next instruction rewrote).  So the row offset joins the lane offset and the scalar
// offset is the constant 0, which makes the compiler keep the wait state.
template <int AUX = 0>
__device__ __forceinline__ void buf_st128(const uint4& w, BufRsrc r, uint32_t voff, uint32_t soff) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  const v4 v = {w.x, w.y, w.z, w.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, int(voff + soff), 0, AUX);
}
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
template <int AUX = 0>
__device__ __forceinline__ void buf_st64(uint32_t lo, uint32_t hi, BufRsrc r, uint32_t voff, uint32_t soff) {
  typedef uint32_t v2 __attribute__((ext_vector_type(2)));
  const v2 v = {lo, hi};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, int(voff), soffset(soff), AUX);
}

// ---- XCD-aware block order --------------------------------------------------------------
// The dispatcher hands consecutive workgroups of a launch to the 8 XCDs in turn, and each XCD
// has its own L2.  Renumbering so that XCD x runs a contiguous range of logical blocks, in
// order, keeps neighbouring blocks (which share parameter rows) on one L2.  Returns the
// logical (x, y) of this block in a 2-D grid; blocks past the largest multiple of 8 keep
// their own index.  Correct for any mapping; only the locality assumes 8 XCDs.
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_remap(uint32_t lin, uint32_t n) {
  const uint32_t per = n / kXcds;
  return lin < per * kXcds ? (lin % kXcds) * per + lin / kXcds : lin;
}
__device__ __forceinline__ void xcd_block(uint32_t& bx, uint32_t& by) {
  const uint32_t gx = gridDim.x;
  const uint32_t lin = xcd_remap(blockIdx.x + blockIdx.y * gx, gx * gridDim.y);
  by = lin / gx;
  bx = lin - by * gx;
}

// ---- quad-lane exchanges through DPP (no LDS traffic) ----------------------------------------
__device__ __forceinline__ float dpp_xor1(float v) {   // quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {   // quad_perm [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// row_half_mirror: lane i of each group of 8 reads lane 7 - i, in the other quad; after the two
// quad exchanges it completes a reduction over 8 consecutive lanes.
__device__ __forceinline__ float dpp_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
}

// row_ror:8: lane i of each row of 16 reads lane (i + 8) mod 16, i.e. lane i ^ 8.
__device__ __forceinline__ float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}

// ---- nontemporal (streaming) global accesses ----------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, const uint4& w) {
  const u32x4 v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ uint32_t ld_stream32(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ void st_stream32(void* p, uint32_t w) {
  __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(p));
}

// ---- inverse map at 64-position granularity ---------------------------------------------
// tile_start[t] = number of rows < 64t.  Called once per compact row j: it writes the
// entries of the tiles whose first listed position is rows[j] (the t with
// rows[j-1] < 64t <= rows[j]), and the row n-1 also writes n for every later tile.  Each
// entry is written by exactly one row; entries are clamped to the array.
// A window of an appended stream covers positions [pos0, pos0 + T): rows hold absolute
// positions, tile t of the window is entry t of tile_start (the caller offsets it), and the
// stream already holds row0 rows before the window, so every entry is offset by row0.
// The same from the window positions p = rows[j] - pos0 and q = rows[j-1] - pos0 (q = -1 for
// j == 0), for a caller that already holds them.
__device__ __forceinline__ void write_tile_index_pq(int32_t p, int32_t q, int32_t n, int32_t T, int32_t j,
                                                    int32_t* __restrict__ tile_start, int32_t row0) {
  const int32_t ntiles = (T + kGroup - 1) / kGroup;
  if (p < 0 || p >= T) return;
  const int32_t t_first = q < 0 ? 0 : min(q / kGroup + 1, ntiles + 1);
  const int32_t t_last = p / kGroup;
  for (int32_t t = t_first; t <= t_last; ++t) tile_start[t] = row0 + j;
  if (j == n - 1)
    for (int32_t t = t_last + 1; t <= ntiles; ++t) tile_start[t] = row0 + n;
}
__device__ __forceinline__ void write_tile_index(const int32_t* __restrict__ rows, int32_t n,
                                                 int32_t T, int32_t j,
                                                 int32_t* __restrict__ tile_start,
                                                 int32_t pos0, int32_t row0) {
  write_tile_index_pq(rows[j] - pos0, j > 0 ? rows[j - 1] - pos0 : -1, n, T, j, tile_start, row0);
}

// lower_bound over an ascending array, computed by a whole 256-thread block in
// ceil(log256(n)) rounds of one parallel probe each (instead of log2(n) dependent loads):
// each round probes 256 evenly spaced entries of the current bracket and keeps the one
// stride that contains the first entry >= key.  Every thread returns the same value.
// Contains __syncthreads_count(); call from all threads of the block.
__device__ __forceinline__ int32_t block_lower_bound(const int32_t* __restrict__ rows, int32_t n,
                                                     int32_t key) {
  int32_t a = 0, b = n;                    // the answer lies in [a, b]
  while (a < b) {
    const int32_t s = (b - a + 255) / 256;
    const int32_t idx = a + int32_t(threadIdx.x) * s;
    const bool pred = idx < b && rows[idx] < key;
    const int32_t c = __syncthreads_count(pred);
    if (c == 0) return a;
    const int32_t na = a + (c - 1) * s + 1;
    const int32_t nb = min(a + c * s, b);
    if (s == 1) return nb;
    a = na;
    b = nb;
  }
  return a;
}


}  // namespace flk
