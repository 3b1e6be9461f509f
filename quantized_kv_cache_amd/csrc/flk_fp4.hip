// flk_fp4.hip -- the NVFP4 variant of the codec (vllm-rlt pull request #166, review item 2:
// E2M1 codes, one E4M3 scale per 16 elements, one FP32 scale per tensor; an INT4 base with
// NVFP4 residuals allowed), on the residual chain of the FlashLoop RFC (section 3.3).
//
//   fp4_amax_kernel<RESID>   the stream's largest magnitude (X, or the BF16 residual against
//                            the reconstruction) into the params header, one atomic per block
//   fp4_encode_kernel<RESID> one thread per 16-channel block: block scale, codes, the decoded
//                            values into the reconstruction, and (compact loops) the tile index
//   fp4_reconstruct_kernel   X_hat from a chain whose base is INT4 or NVFP4 and whose residual
//                            loops are NVFP4; a block per (64-position tile, slice of blocks)
//
// Element formats: E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7, sign in bit 3);
// E4M3 bias 7, subnormal below 2^-6 (steps of 2^-9), largest finite 448.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "flk_device.h"
#include "flk_fp4.h"
#include "flk_internal.h"

namespace flk {

namespace {

constexpr int kFp4Threads = 256;
constexpr int kAmaxBlocks = 1024;
constexpr int kRecItemsPerThread = 4;

// ---- element formats ------------------------------------------------------------------------

// Nearest-even E4M3 of a non-negative finite v, saturated at 448: the value, and its byte.
__device__ __forceinline__ float e4m3_round(float v, uint32_t& byte) {
  if (v >= 448.0f) {
    byte = 0x7Eu;
    return 448.0f;
  }
  if (v < 0x1p-6f) {                                   // subnormal grid, steps of 2^-9
    const float q = __builtin_rintf(v * 512.0f);       // exact scaling; q in 0..8
    byte = uint32_t(q);
    return q * 0x1p-9f;
  }
  const int e = int((__float_as_uint(v) >> 23) & 0xFFu) - 127;
  const float q = __builtin_rintf(__builtin_ldexpf(v, 3 - e));   // 8..16 (16: next binade)
  byte = (uint32_t(e + 7) << 3) + uint32_t(q) - 8u;
  return __builtin_ldexpf(q, e - 3);
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e == 0 ? float(m) * 0x1p-9f : __builtin_ldexpf(1.0f + float(m) * 0.125f, int(e) - 7);
}

// E2M1 magnitude 0..7 -> value.
__device__ __forceinline__ float e2m1_value(uint32_t mag) {
  return mag < 2 ? 0.5f * float(mag) : __uint_as_float((((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22));
}

// Magnitude code of the nearest-even E2M1 value to |y| = a, saturated at 6; the grid step is
// 0.5 below 2, 1 below 4, 2 above, so a / step is exact and rint picks the even neighbour.
__device__ __forceinline__ float e2m1_steps(float a, float& step) {
  step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
  return a * (1.0f / step);
}
__device__ __forceinline__ uint32_t e2m1_mag_of(float k, float step) {
  if (step == 0.5f) return uint32_t(k);                          // 0..4
  if (step == 1.0f) return uint32_t(k) + 2u;                     // 2..4 -> 4..6
  return uint32_t(__builtin_fminf(k, 3.0f)) + 4u;                // 2, 3, >= 4 -> 6, 7, 7
}

// Code (sign in bit 3) of v against the block's scale bs > 0 with rbs ~ 1/bs.  Fast path:
// q = RN(v * rbs) is within 3 ulp of RN(v / bs); with |v| <= 6.4 bs, |q| / step stays below
// 13, so its rounding can differ from that of the exact quotient only within 2^-15 of a
// half-integer, where the correctly rounded division decides (as it does when q is not a
// finite value below 16 steps, e.g. when a tiny bs has no finite reciprocal).
__device__ __forceinline__ uint32_t e2m1_code(float v, float bs, float rbs) {
  float step;
  float t = e2m1_steps(__builtin_fabsf(v * rbs), step);
  float k = __builtin_rintf(t);
  if (__builtin_expect(!(t < 16.0f) || __builtin_fabsf(t - k) > 0.5f - 0x1p-15f, 0)) {
    t = e2m1_steps(__builtin_fabsf(v / bs), step);
    k = __builtin_rintf(t);
  }
  return e2m1_mag_of(k, step) | (__builtin_signbit(v) ? 8u : 0u);
}

__device__ __forceinline__ float e2m1_decode(uint32_t code, float bs) {
  const float m = e2m1_value(code & 7u) * bs;
  return (code & 8u) ? -m : m;
}

// Stream scale from the stream's largest magnitude.
__device__ __forceinline__ float stream_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 2688.0f; }

// ---- stream amax ----------------------------------------------------------------------------

// 8 magnitudes (16 bytes of BF16) of chunk c of the stream: x itself, or the BF16 residual
// against the reconstruction at the chunk's position.
template <bool RESID>
__device__ __forceinline__ void chunk_values(const uint16_t* __restrict__ x, const int32_t* __restrict__ rows,
                                             const uint16_t* __restrict__ recon, int32_t W, int64_t c,
                                             float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(x + 8 * c);
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(wa[i]);
    v[2 * i + 1] = bf16_hi(wa[i]);
  }
  if (RESID) {
    const int64_t e = 8 * c;
    const int64_t j = e / W;
    const int64_t p = rows ? rows[j] : j;
    const uint4 b = *reinterpret_cast<const uint4*>(recon + p * W + (e - j * W));
    const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = round_bf16(v[2 * i] - bf16_lo(wb[i]));
      v[2 * i + 1] = round_bf16(v[2 * i + 1] - bf16_hi(wb[i]));
    }
  }
}

template <bool RESID>
__global__ __launch_bounds__(kFp4Threads) void fp4_amax_kernel(const uint16_t* __restrict__ x,
                                                                 const int32_t* __restrict__ rows,
                                                                 const uint16_t* __restrict__ recon, int64_t chunks,
                                                                 int32_t W, uint32_t* __restrict__ amax_word,
                                                                 uint32_t* __restrict__ status) {
  __shared__ float wmax[kFp4Threads / 64];
  float m = 0.0f;
  bool bad = false;
  for (int64_t c = int64_t(blockIdx.x) * kFp4Threads + threadIdx.x; c < chunks;
       c += int64_t(gridDim.x) * kFp4Threads) {
    float v[8];
    chunk_values<RESID>(x, rows, recon, W, c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bad |= !__builtin_isfinite(v[i]);
      m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
    }
  }
  if (bad && status) atomicOr(status, FLK_DEV_NONFINITE);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kFp4Threads / 64; ++i) m = __builtin_fmaxf(m, wmax[i]);
    if (m > 0.0f) atomicMax(amax_word, __float_as_uint(m));   // non-negative floats order as integers
  }
}

// ---- encode ----------------------------------------------------------------------------------

template <bool RESID>
__global__ __launch_bounds__(kFp4Threads) void fp4_encode_kernel(const uint16_t* __restrict__ x,
                                                                  const int32_t* __restrict__ rows,
                                                                  uint16_t* __restrict__ recon, int32_t n, int32_t T,
                                                                  int32_t W, uint8_t* __restrict__ codes,
                                                                  uint32_t* __restrict__ params,
                                                                  int32_t* __restrict__ tile_start) {
  const int32_t bpr = W / 16;                                     // blocks per row
  const int64_t i = int64_t(blockIdx.x) * kFp4Threads + threadIdx.x;
  const float s_g = stream_scale(__uint_as_float(params[1]));
  if (i == 0) {
    params[0] = __float_as_uint(s_g);
    params[2] = 0u;
    params[3] = 0u;
  }
  if (i >= int64_t(n) * bpr) return;
  const int32_t j = int32_t(i / bpr);
  const int32_t rem = int32_t(i - int64_t(j) * bpr);
  if (RESID && rows && rem == 0) write_tile_index(rows, n, T, j, tile_start, 0, 0);
  float v[16], prev[16];
  uint16_t* dst;
  {
    const uint4 a0 = *reinterpret_cast<const uint4*>(x + 16 * i);
    const uint4 a1 = *reinterpret_cast<const uint4*>(x + 16 * i + 8);
    const uint32_t wa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[2 * e] = bf16_lo(wa[e]);
      v[2 * e + 1] = bf16_hi(wa[e]);
    }
  }
  if (RESID) {
    const int64_t p = rows ? rows[j] : j;
    dst = recon + p * W + 16 * rem;
    const uint4 b0 = *reinterpret_cast<const uint4*>(dst);
    const uint4 b1 = *reinterpret_cast<const uint4*>(dst + 8);
    const uint32_t wb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      prev[2 * e] = bf16_lo(wb[e]);
      prev[2 * e + 1] = bf16_hi(wb[e]);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = round_bf16(v[e] - prev[e]);   // the residual, in BF16
  } else {
    dst = recon + 16 * i;
  }
  float amax_b = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(v[e]));
  uint32_t sbyte;
  const float e4 = e4m3_round(amax_b / (6.0f * s_g), sbyte);
  const float bs = e4 * s_g;
  const float rbs = __builtin_amdgcn_rcpf(bs);
  uint32_t cw[2] = {0u, 0u};
  float dec[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t c = bs > 0.0f ? e2m1_code(v[e], bs, rbs) : 0u;
    cw[e >> 3] |= c << (4 * (e & 7));
    dec[e] = e2m1_decode(c, bs);
  }
  *reinterpret_cast<uint2*>(codes + 8 * i) = make_uint2(cw[0], cw[1]);
  reinterpret_cast<uint8_t*>(params)[16 + i] = uint8_t(sbyte);
  uint32_t o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (RESID) {
      const float d0 = round_bf16(dec[2 * e]), d1 = round_bf16(dec[2 * e + 1]);
      o[e] = pack_bf16x2(prev[2 * e] + d0, prev[2 * e + 1] + d1);
    } else {
      o[e] = pack_bf16x2(dec[2 * e], dec[2 * e + 1]);
    }
  }
  *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint4*>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
}

// ---- reconstruct (mixed chains) -------------------------------------------------------------

// Block (tile, part): items part*1024 .. of the tile, item = (position in tile, 16-channel
// block of the row); thread tid takes items part*1024 + k*256 + tid, k < 4, so consecutive
// threads write consecutive 32-byte pieces of a row.  Compact loops map the tile's positions
// to their compact rows through an LDS table built from the tile index.
__global__ __launch_bounds__(kFp4Threads) void fp4_reconstruct_kernel(ChainArgs c, int32_t base_fp4, int32_t kind,
                                                                       int32_t T, int32_t H, int32_t D,
                                                                       uint16_t* __restrict__ out) {
  __shared__ int32_t lmap[FLK_MAX_LOOPS][kGroup];
  const int32_t tile = blockIdx.x;
  const int32_t W = H * D, bpr = W / 16, bph = D / 16;
  const int tid = threadIdx.x;
  for (int l = 1; l < c.n_loops; ++l) {
    if (!c.s[l].rows) continue;
    if (tid < kGroup) lmap[l][tid] = -1;
  }
  __syncthreads();
  for (int l = 1; l < c.n_loops; ++l) {
    const StreamArgs& s = c.s[l];
    if (!s.rows) continue;
    const int32_t j0 = s.tile_start[tile], j1 = s.tile_start[tile + 1];
    if (tid < j1 - j0) {
      const int32_t p = s.rows[j0 + tid] - tile * kGroup;
      if (p >= 0 && p < kGroup) lmap[l][p] = j0 + tid;
    }
  }
  __syncthreads();
  const int32_t items = kGroup * bpr;
  for (int k = 0; k < kRecItemsPerThread; ++k) {
    const int32_t item = int32_t(blockIdx.y) * (kRecItemsPerThread * kFp4Threads) + k * kFp4Threads + tid;
    if (item >= items) break;
    const int32_t pl = item / bpr, blk = item - pl * bpr;
    const int32_t p = tile * kGroup + pl;
    if (p >= T) break;
    const int32_t h = blk / bph, c0 = 16 * (blk - h * bph);
    const int64_t off = int64_t(p) * W + int64_t(h) * D + c0;    // element offset in [T, H, D]
    float x[16];
    const StreamArgs& b = c.s[0];
    const uint2 bc = *reinterpret_cast<const uint2*>(b.codes + off / 2);
    const uint32_t bw[2] = {bc.x, bc.y};
    if (base_fp4) {
      const float s_g = __uint_as_float(b.params[0]);
      const float bs = e4m3_value(reinterpret_cast<const uint8_t*>(b.params)[16 + int64_t(p) * bpr + blk]) * s_g;
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = round_bf16(e2m1_decode((bw[e >> 3] >> (4 * (e & 7))) & 15u, bs));
    } else if (kind == FLK_KIND_K) {                            // one (min, scale) per channel of the 64-row group
      const uint32_t* pk = b.params + int64_t(p / kGroup) * W + int64_t(h) * D + c0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 pw = *reinterpret_cast<const uint4*>(pk + 4 * q);
        const uint32_t pa[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ch = 4 * q + e;
          const float code = float((bw[ch >> 3] >> (4 * (ch & 7))) & 15u);
          x[ch] = round_bf16(decode(code, f16_bits_to_f32(pa[e] & 0xFFFFu), f16_bits_to_f32(pa[e] >> 16)));
        }
      }
    } else {                                                    // V: one (min, scale) per 64 channels
      const uint32_t pv = b.params[(int64_t(p) * H + h) * ((D + kGroup - 1) / kGroup) + c0 / kGroup];
      const float mn = f16_bits_to_f32(pv & 0xFFFFu), sc = f16_bits_to_f32(pv >> 16);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = round_bf16(decode(float((bw[e >> 3] >> (4 * (e & 7))) & 15u), mn, sc));
    }
    for (int l = 1; l < c.n_loops; ++l) {
      const StreamArgs& s = c.s[l];
      const int32_t j = s.rows ? lmap[l][pl] : p;
      if (j < 0) continue;                                      // inherits
      const int64_t roff = int64_t(j) * W + int64_t(h) * D + c0;
      const uint2 rc = *reinterpret_cast<const uint2*>(s.codes + roff / 2);
      const uint32_t rw[2] = {rc.x, rc.y};
      const float s_g = __uint_as_float(s.params[0]);
      const float bs = e4m3_value(reinterpret_cast<const uint8_t*>(s.params)[16 + int64_t(j) * bpr + blk]) * s_g;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        x[e] = round_bf16(x[e] + round_bf16(e2m1_decode((rw[e >> 3] >> (4 * (e & 7))) & 15u, bs)));
    }
    uint16_t* o = out + off;
    *reinterpret_cast<uint4*>(o) = pack_exact_bf16x8(x);
    *reinterpret_cast<uint4*>(o + 8) = pack_exact_bf16x8(x + 8);
  }
}

}  // namespace

hipError_t launch_fp4_encode(bool resid, const void* x, const int32_t* rows, int32_t n, int32_t T, int32_t H,
                             int32_t D, void* recon, uint8_t* codes, uint32_t* params, int32_t* tile_start,
                             uint32_t* status, hipStream_t stream) {
  const int32_t W = H * D;
  if (D % 16 != 0 || n < 1) return hipErrorInvalidValue;
  hipError_t e = launch_fill_u32(params + 1, 1, 0u, stream);           // the header's amax word
  if (e != hipSuccess) return e;
  const int64_t chunks = int64_t(n) * W / 8;
  const unsigned ab = unsigned(std::min<int64_t>(kAmaxBlocks, (chunks + kFp4Threads - 1) / kFp4Threads));
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* rc = static_cast<uint16_t*>(recon);
  const unsigned eb = unsigned((int64_t(n) * (W / 16) + kFp4Threads - 1) / kFp4Threads);
  if (resid) {
    hipLaunchKernelGGL(fp4_amax_kernel<true>, dim3(ab), dim3(kFp4Threads), 0, stream, xs, rows, rc, chunks, W,
                       params + 1, status);
    hipLaunchKernelGGL(fp4_encode_kernel<true>, dim3(eb), dim3(kFp4Threads), 0, stream, xs, rows, rc, n, T, W,
                       codes, params, tile_start);
  } else {
    hipLaunchKernelGGL(fp4_amax_kernel<false>, dim3(ab), dim3(kFp4Threads), 0, stream, xs, rows, rc, chunks, W,
                       params + 1, status);
    hipLaunchKernelGGL(fp4_encode_kernel<false>, dim3(eb), dim3(kFp4Threads), 0, stream, xs, rows, rc, n, T, W,
                       codes, params, tile_start);
  }
  return hipGetLastError();
}

hipError_t launch_fp4_reconstruct(const ChainArgs& chain, bool base_fp4, int kind, int32_t T, int32_t H, int32_t D,
                                  void* out, hipStream_t stream) {
  if (D % 16 != 0 || chain.n_loops < 1) return hipErrorInvalidValue;
  const int32_t items = kGroup * (H * D / 16);
  const unsigned parts = unsigned((items + kRecItemsPerThread * kFp4Threads - 1) / (kRecItemsPerThread * kFp4Threads));
  const dim3 grid(unsigned((T + kGroup - 1) / kGroup), parts);
  hipLaunchKernelGGL(fp4_reconstruct_kernel, grid, dim3(kFp4Threads), 0, stream, chain, base_fp4 ? 1 : 0, kind, T,
                     H, D, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace flk
