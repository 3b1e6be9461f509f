// hw_arith_check.hip -- exhaustive checks of gfx950 arithmetic facts the kernels rely on: two for
// the exact K decode of the decode-attention scores kernel, one for the encoders.  Test infrastructure: built by build(), run by
// tests/test_gpu_hw_arith.py; the library does not use this file.
//
// 1. v_dot2_f32_bf16 (a, b) . (1, 1) + 0, rounded to BF16 by v_cvt_pk_bf16_f32, equals the BF16
//    rounding of v_add_f32 (a, b), for every pair of BF16 values that are +0 or finite and
//    normal (the chain's values: multiples of 2^-24, never -0).  The dot's binary32 result is
//    not always the correctly rounded sum when the two exponents are 16 or more apart, but then
//    the sum lies far from any BF16 rounding boundary, so the BF16 result is the same.
// 2. v_fma_mix_f32 with a binary16 operand holding a 4-bit code as its bit pattern (the
//    denormal code * 2^-24) times s * 2^24 in binary32 plus a binary16 minimum m equals
//    fma(code, s, m) in binary32, for every finite non-negative binary16 scale s, every code
//    and 512 minima (zeros, denormals, both signs, the extremes).
// 3. The encoders' three-instruction RN(x / 15) (flk::div15) equals the IEEE division for every
//    finite binary32 x >= +0, denormals included.
// 4. v_cvt_scalef32_pk_f32_fp8 with scale 1 (flk::e4m3x2_value), either 16-bit half, gives
//    flk::fp4_e4m3_value of both bytes for every pair of non-negative finite E4M3 bytes (the
//    NVFP4 block scales the decode-attention readers convert with it).
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>

#include "../../quantized_kv_cache_amd/csrc/flk_device.h"
#include "../../quantized_kv_cache_amd/csrc/flk_fp4_device.h"

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const f32x2 v = {x, 0.0f};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2)) & 0xFFFFu;
}
__device__ __forceinline__ bool in_domain(uint32_t v) {       // +0, or finite and normal
  const uint32_t e = (v >> 7) & 0xFFu;
  return v == 0u || (e != 0u && e != 0xFFu);
}

// grid 65536 x 256: block a, thread t covers b = 256 t .. 256 t + 255
__global__ void check_dot2(const uint32_t* ones_in, unsigned long long* cnt) {
  const uint32_t a = blockIdx.x;
  const uint32_t ones = ones_in[0];
  unsigned long long bad = 0, inexact_close = 0, tested = 0;
  if (in_domain(a)) {
    for (uint32_t i = 0; i < 256; ++i) {
      const uint32_t b = threadIdx.x * 256u + i;
      if (!in_domain(b)) continue;
      float r1;
      // the 3 wait states a VALU read of the dot's result needs, as in the kernel's asm
      asm volatile("v_dot2_f32_bf16 %0, %1, %2, 0\n\ts_nop 2" : "=v"(r1) : "v"((b << 16) | a), "s"(ones));
      const float r2 = __uint_as_float(a << 16) + __uint_as_float(b << 16);
      ++tested;
      if (bf16_rne(r1) != bf16_rne(r2)) ++bad;
      const int ea = int((a >> 7) & 0xFFu), eb = int((b >> 7) & 0xFFu);
      const int de = ea > eb ? ea - eb : eb - ea;
      if (a != 0u && b != 0u && de < 16 && __float_as_uint(r1) != __float_as_uint(r2)) ++inexact_close;
    }
  }
  atomicAdd(&cnt[0], tested);
  if (bad) atomicAdd(&cnt[1], bad);
  if (inexact_close) atomicAdd(&cnt[2], inexact_close);
}

// grid 0x7C00 x 512: block = binary16 scale bits, thread = index of the minimum
__global__ void check_fma_mix(const uint16_t* ms, unsigned long long* cnt) {
  const uint32_t s16 = blockIdx.x;
  const uint32_t m16 = ms[threadIdx.x];
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)s16);
  const float sp = s * 16777216.0f;
  const float m = (float)__builtin_bit_cast(_Float16, (uint16_t)m16);
  unsigned long long bad = 0;
  for (uint32_t c0 = 0; c0 < 16; ++c0) {
    uint32_t code = c0;
    asm volatile("" : "+v"(code));              // a run-time value
    float r1;
    asm volatile("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,1]" : "=v"(r1) : "v"(code), "v"(sp), "v"(m16));
    const float r2 = __builtin_fmaf((float)code, s, m);
    if (__float_as_uint(r1) != __float_as_uint(r2)) ++bad;
  }
  atomicAdd(&cnt[3], 16ull);
  if (bad) atomicAdd(&cnt[4], bad);
}

// grid-stride over every finite binary32 x >= +0: div15 (the params' RN(x / 15)) against the
// IEEE division
__global__ void check_div15(unsigned long long* cnt) {
  unsigned long long bad = 0, tested = 0;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < 0x7F800000u; u += stride) {
    float x = __uint_as_float(u);
    asm volatile("" : "+v"(x));                 // a run-time value
    const float q1 = flk::div15(x);
    const float q2 = x / 15.0f;
    ++tested;
    if (__float_as_uint(q1) != __float_as_uint(q2)) ++bad;
  }
  atomicAdd(&cnt[5], tested);
  if (bad) atomicAdd(&cnt[6], bad);
}

// grid 256 x 256: block a, thread t checks bytes (a, t) in both halves of the word
__global__ void check_e4m3(unsigned long long* cnt) {
  const uint32_t b0 = blockIdx.x, b1 = threadIdx.x;
  if (b0 >= 0x7Fu || b1 >= 0x7Fu) return;       // non-negative finite bytes only (0x7F is NaN)
  uint32_t w = b0 | (b1 << 8) | (b0 << 16) | (b1 << 24);
  asm volatile("" : "+v"(w));                   // a run-time value
  const flk::fp4_f32x2 lo = flk::e4m3x2_value<false>(w), hi = flk::e4m3x2_value<true>(w);
  const float e0 = flk::fp4_e4m3_value(b0), e1 = flk::fp4_e4m3_value(b1);
  const bool ok = __float_as_uint(lo.x) == __float_as_uint(e0) && __float_as_uint(lo.y) == __float_as_uint(e1) &&
                  __float_as_uint(hi.x) == __float_as_uint(e0) && __float_as_uint(hi.y) == __float_as_uint(e1);
  atomicAdd(&cnt[7], 1ull);
  if (!ok) atomicAdd(&cnt[8], 1ull);
}

int main() {
  uint16_t hm[512];
  uint32_t x = 12345u;
  for (int i = 0; i < 512; ++i) {
    x = x * 1664525u + 1013904223u;
    uint16_t v = uint16_t(x >> 16);
    if ((v & 0x7C00u) == 0x7C00u) v &= 0xBFFFu;   // no Inf / NaN
    hm[i] = v;
  }
  hm[0] = 0x0000; hm[1] = 0x8000; hm[2] = 0x0001; hm[3] = 0x8001; hm[4] = 0x03FF; hm[5] = 0x7BFF; hm[6] = 0xFBFF;
  uint32_t* ones = nullptr;
  uint16_t* ms = nullptr;
  unsigned long long* cnt = nullptr;
  const uint32_t one2 = 0x3F803F80u;
  if (hipMalloc(&ones, 4) != hipSuccess || hipMalloc(&ms, sizeof(hm)) != hipSuccess ||
      hipMalloc(&cnt, 8 * 9) != hipSuccess || hipMemcpy(ones, &one2, 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ms, hm, sizeof(hm), hipMemcpyHostToDevice) != hipSuccess || hipMemset(cnt, 0, 8 * 9) != hipSuccess) {
    printf("setup failed\n");
    return 2;
  }
  hipLaunchKernelGGL(check_dot2, dim3(65536), dim3(256), 0, 0, ones, cnt);
  hipLaunchKernelGGL(check_fma_mix, dim3(0x7C00), dim3(512), 0, 0, ms, cnt);
  hipLaunchKernelGGL(check_div15, dim3(65536), dim3(256), 0, 0, cnt);
  hipLaunchKernelGGL(check_e4m3, dim3(256), dim3(256), 0, 0, cnt);
  unsigned long long c[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(c, cnt, 8 * 9, hipMemcpyDeviceToHost) != hipSuccess) {
    printf("run failed\n");
    return 2;
  }
  printf("dot2_pairs %llu dot2_bf16_mismatch %llu dot2_inexact_below_16 %llu\n", c[0], c[1], c[2]);
  printf("fma_mix_cases %llu fma_mix_mismatch %llu\n", c[3], c[4]);
  printf("div15_cases %llu div15_mismatch %llu\n", c[5], c[6]);
  printf("e4m3_pairs %llu e4m3_mismatch %llu\n", c[7], c[8]);
  return (c[1] == 0 && c[4] == 0 && c[6] == 0 && c[8] == 0) ? 0 : 1;
}
