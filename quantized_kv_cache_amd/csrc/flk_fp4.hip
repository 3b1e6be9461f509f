// flk_fp4.hip -- the FP4 variants of the codec on the residual chain of the FlashLoop RFC
// (section 3.3): NVFP4 (vllm-rlt pull request #166, review item 2: E2M1 codes, one E4M3 scale
// per 16 elements, one FP32 scale per tensor; an INT4 base with NVFP4 residuals allowed) and
// MXFP4 (OCP Microscaling Formats v1.0, section 6: E2M1 codes, one E8M0 power-of-two scale per
// 32 elements, no tensor scale).
//
//   fp4_amax_kernel<RESID>       NVFP4: per-block maxima of the stream's magnitudes (X, or the
//                                BF16 residual against the reconstruction), parked in the
//                                stream's codes buffer, which the encoder overwrites afterwards
//   fp4_amax_fold_kernel         NVFP4: their maximum into the params header
//   fp4_encode_kernel<RESID, MX> lanes own 8 channels of a 16-channel (NVFP4) or 32-channel
//                                (MXFP4) block: block scale, codes, the decoded values into the
//                                reconstruction, and (compact loops) the tile index
//   fp4_reconstruct_kernel       X_hat from a chain whose base is INT4 or FP4 and whose residual
//                                loops are FP4 of one kind; a block per (64-position tile,
//                                slice of 16-channel items)
//
// Element formats: E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7, sign in bit 3);
// E4M3 bias 7, subnormal below 2^-6 (steps of 2^-9), largest finite 448; E8M0 a bare biased
// exponent, byte b = 2^(b - 127).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "flk_device.h"
#include "flk_fp4.h"
#include "flk_fp4_device.h"
#include "flk_internal.h"

namespace flk {

namespace {

constexpr int kFp4Threads = 256;
constexpr int kAmaxBlocks = 1024;
constexpr int kAmaxUnroll = 4;
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


// gfx950 converts pairs of binary32 values to E2M1 codes (v_cvt_scalef32_pk_fp4_f32) and back
// (v_cvt_scalef32_pk_f32_fp4).  With a scale of 1 the conversion to E2M1 is the nearest-even
// value, saturated at 6, with the sign kept for values that round to zero (zeros and
// subnormals included), and the conversion back is exact -- checked against the oracle's
// rounding on ties, their neighbours, saturation, signed zeros and subnormals.  (A scale that
// is not a power of two contributes only its exponent, so the block scale is divided out
// beforehand.)  Pair k of a word is byte k; its low nibble is the even element.
__device__ __forceinline__ uint32_t cvt_pair(uint32_t w, float a, float b, int k) {
  switch (k) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 3);
  }
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 uncvt_pair(uint32_t w, int k) {
  switch (k) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// Codes of 8 values (4 pairs, one word) against the block's scale bs > 0, and their decoded
// values RN32(e2m1 * bs).  The code of v is the E2M1 rounding of y = RN32(v / bs).  Fast path:
// q = RN(v * rcp(bs)) lies within 2^-22 (relative) of y for a normal bs, so y lies between
// q (1 - 2^-21) and q (1 + 2^-21); E2M1 rounding is monotonic, so when both ends give the
// same codes, y does too.  Otherwise (or for a bs outside the normal range) the correctly
// rounded division decides.
__device__ __forceinline__ uint32_t e2m1_encode8(const float v[8], float bs, float dec[8]) {
  uint32_t cw = 0u;
  bool exact = !(bs >= 0x1p-126f && bs <= 0x1p125f);
  if (!exact) {
    const float rbs = __builtin_amdgcn_rcpf(bs);
    const float lo = 1.0f - 0x1p-21f, hi = 1.0f + 0x1p-21f;
    uint32_t clo = 0u, chi = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float q0 = v[2 * k] * rbs, q1 = v[2 * k + 1] * rbs;
      clo = cvt_pair(clo, q0 * lo, q1 * lo, k);
      chi = cvt_pair(chi, q0 * hi, q1 * hi, k);
    }
    cw = clo;
    exact = clo != chi;
  }
  if (__builtin_expect(exact, 0)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) cw = cvt_pair(cw, v[2 * k] / bs, v[2 * k + 1] / bs, k);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 d = uncvt_pair(cw, k);
    dec[2 * k] = d.x * bs;
    dec[2 * k + 1] = d.y * bs;
  }
  return cw;
}


// MXFP4 shared scale of a block from its largest magnitude: floor(log2 amax) - 2 (E2M1's
// largest power of two is 2^2), clamped to E8M0's smallest exponent -127; the biased byte is
// the exponent field of amax less 2, or 0 (amax zero, subnormal, or below 2^-124).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
  return ef > 2u ? ef - 2u : 0u;
}

// Codes of 8 values against an MXFP4 block scale 2^(byte - 127), and their decoded values.
// The quotient x / X is x times the power of two 2^(127 - byte) (a normal binary32 for every
// byte up to 252), exact except where it falls below 2^-126, far under the smallest E2M1
// rounding boundary 0.25, where the code is a signed zero either way.
__device__ __forceinline__ uint32_t mx_encode8(const float v[8], uint32_t byte, float dec[8]) {
  const float inv = __uint_as_float((254u - byte) << 23);
  const float X = fp4_e8m0_value(byte);
  uint32_t cw = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) cw = cvt_pair(cw, v[2 * k] * inv, v[2 * k + 1] * inv, k);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 d = uncvt_pair(cw, k);
    dec[2 * k] = d.x * X;
    dec[2 * k + 1] = d.y * X;
  }
  return cw;
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
                                                                 int32_t W, float* __restrict__ partial,
                                                                 uint32_t* __restrict__ status) {
  __shared__ float wmax[kFp4Threads / 64];
  float m = 0.0f;
  bool bad = false;
  const int64_t stride = int64_t(gridDim.x) * kFp4Threads;
  for (int64_t c0 = int64_t(blockIdx.x) * kFp4Threads + threadIdx.x; c0 < chunks; c0 += kAmaxUnroll * stride) {
    float v[kAmaxUnroll][8];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {           // kAmaxUnroll chunks in flight per thread
      const int64_t c = c0 + u * stride;
      if (c < chunks) {
        chunk_values<RESID>(x, rows, recon, W, c, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bad |= !__builtin_isfinite(v[u][i]);
        m = __builtin_fmaxf(m, __builtin_fabsf(v[u][i]));
      }
  }
  if (bad && status) atomicOr(status, FLK_DEV_NONFINITE);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kFp4Threads / 64; ++i) m = __builtin_fmaxf(m, wmax[i]);
    partial[blockIdx.x] = m;
  }
}

// The stream amax from the blocks' maxima, into the header's amax word.
__global__ __launch_bounds__(kFp4Threads) void fp4_amax_fold_kernel(const float* __restrict__ partial, int32_t nb,
                                                                     uint32_t* __restrict__ params) {
  __shared__ float wmax[kFp4Threads / 64];
  float m = 0.0f;
  for (int32_t i = threadIdx.x; i < nb; i += kFp4Threads) m = __builtin_fmaxf(m, partial[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kFp4Threads / 64; ++i) m = __builtin_fmaxf(m, wmax[i]);
    params[1] = __float_as_uint(m);
  }
}

// ---- encode ----------------------------------------------------------------------------------

// NVFP4: lane pairs own a 16-channel block: lane 2m holds its channels 0..7, lane 2m+1
// channels 8..15 (16 coalesced bytes per lane and tensor), and the pair takes the block's amax
// with one shuffle.  MXFP4: lane quads own a 32-channel block, two shuffles.  Each lane writes
// its 4 bytes of codes and 16 bytes of reconstruction; the block's first lane its scale byte.
// The NVFP4 amax pass reports non-finite inputs; the MXFP4 encoder, which has no such pass,
// checks them itself.
template <bool RESID, bool MX>
__global__ __launch_bounds__(kFp4Threads) void fp4_encode_kernel(const uint16_t* __restrict__ x,
                                                                  const int32_t* __restrict__ rows,
                                                                  uint16_t* __restrict__ recon, int32_t n, int32_t T,
                                                                  int32_t W, uint8_t* __restrict__ codes,
                                                                  uint32_t* __restrict__ params,
                                                                  int32_t* __restrict__ tile_start,
                                                                  uint32_t* __restrict__ status) {
  const int64_t c = int64_t(blockIdx.x) * kFp4Threads + threadIdx.x;    // 8-element chunk
  const float s_g = MX ? 1.0f : stream_scale(__uint_as_float(params[1]));
  if (!MX && c == 0) {
    params[0] = __float_as_uint(s_g);
    params[2] = 0u;
    params[3] = 0u;
  }
  const int64_t chunks = int64_t(n) * (W / 8);
  const bool live = c < chunks;                        // chunks is even: pairs are whole
  const int64_t cc = live ? c : 0;
  const int64_t e0 = 8 * cc;
  const int32_t j = int32_t(e0 / W);
  const int64_t within = e0 - int64_t(j) * W;
  if (RESID && rows && live && within == 0) write_tile_index(rows, n, T, j, tile_start, 0, 0);
  float v[8], prev[8];
  uint16_t* dst;
  {
    const uint4 a = *reinterpret_cast<const uint4*>(x + e0);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(wa[e]);
      v[2 * e + 1] = bf16_hi(wa[e]);
    }
  }
  if (RESID) {
    const int64_t p = rows ? rows[j] : j;
    dst = recon + p * W + within;
    const uint4 b = *reinterpret_cast<const uint4*>(dst);
    const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      prev[2 * e] = bf16_lo(wb[e]);
      prev[2 * e + 1] = bf16_hi(wb[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = round_bf16(v[e] - prev[e]);      // the residual, in BF16
  } else {
    dst = recon + e0;
  }
  float amax_b = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(v[e]));
  amax_b = __builtin_fmaxf(amax_b, __shfl_xor(amax_b, 1));
  if (MX) amax_b = __builtin_fmaxf(amax_b, __shfl_xor(amax_b, 2));
  if (!live) return;
  uint32_t cw = 0u;
  float dec[8];
  if (MX) {
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) bad |= !__builtin_isfinite(v[e]);
    if (bad && status) atomicOr(status, FLK_DEV_NONFINITE);
    const uint32_t sbyte = mx_scale_byte(amax_b);
    cw = mx_encode8(v, sbyte, dec);
    if ((c & 3) == 0) reinterpret_cast<uint8_t*>(params)[c >> 2] = uint8_t(sbyte);
  } else {
    uint32_t sbyte;
    const float e4 = e4m3_round(amax_b / (6.0f * s_g), sbyte);
    const float bs = e4 * s_g;
    if (bs > 0.0f) {
      cw = e2m1_encode8(v, bs, dec);
    } else {                                           // a block whose scale is 0: codes +0
#pragma unroll
      for (int e = 0; e < 8; ++e) dec[e] = 0.0f;
    }
    if ((c & 1) == 0) reinterpret_cast<uint8_t*>(params)[16 + (c >> 1)] = uint8_t(sbyte);
  }
  *reinterpret_cast<uint32_t*>(codes + 4 * c) = cw;
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (RESID)
      o[e] = pack_bf16x2(prev[2 * e] + round_bf16(dec[2 * e]), prev[2 * e + 1] + round_bf16(dec[2 * e + 1]));
    else
      o[e] = pack_bf16x2(dec[2 * e], dec[2 * e + 1]);
  }
  *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ---- reconstruct (mixed chains) -------------------------------------------------------------

// The binary32 scale of the FP4 block holding element offset off (in [n, H, D]) of a stream:
// MXFP4 its E8M0 byte, at off / 32; NVFP4 its E4M3 byte (after the 16-byte header, at 16 +
// off / 16) times the stream scale.
__device__ __forceinline__ float fp4_block_scale(const uint32_t* params, int64_t off, bool mx) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(params);
  if (mx) return fp4_e8m0_value(b[off / 32]);
  return fp4_e4m3_value(b[16 + off / 16]) * __uint_as_float(params[0]);
}

// Block (tile, part): items part*1024 .. of the tile, item = (position in tile, 16-channel
// piece of the row); thread tid takes items part*1024 + k*256 + tid, k < 4, so consecutive
// threads write consecutive 32-byte pieces of a row.  Compact loops map the tile's positions
// to their compact rows through an LDS table built from the tile index.  mx: the FP4 loops
// are MXFP4, else NVFP4.
__global__ __launch_bounds__(kFp4Threads) void fp4_reconstruct_kernel(ChainArgs c, int32_t base_fp4, int32_t mx,
                                                                       int32_t kind, int32_t T, int32_t H, int32_t D,
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
      const float bs = fp4_block_scale(b.params, off, mx != 0);
      fp4_decode8(bw[0], bs, x);
      fp4_decode8(bw[1], bs, x + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = round_bf16(x[e]);
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
      const float bs = fp4_block_scale(s.params, roff, mx != 0);
      float d[16];
      fp4_decode8(rw[0], bs, d);
      fp4_decode8(rw[1], bs, d + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = round_bf16(x[e] + round_bf16(d[e]));
    }
    uint16_t* o = out + off;
    *reinterpret_cast<uint4*>(o) = pack_exact_bf16x8(x);
    *reinterpret_cast<uint4*>(o + 8) = pack_exact_bf16x8(x + 8);
  }
}

}  // namespace

hipError_t launch_fp4_encode(bool resid, bool mx, const void* x, const int32_t* rows, int32_t n, int32_t T,
                             int32_t H, int32_t D, void* recon, uint8_t* codes, uint32_t* params,
                             int32_t* tile_start, uint32_t* status, hipStream_t stream) {
  const int32_t W = H * D;
  if (D % (mx ? 32 : 16) != 0 || n < 1) return hipErrorInvalidValue;
  const int64_t chunks = int64_t(n) * W / 8;
  const auto* xs = static_cast<const uint16_t*>(x);
  auto* rc = static_cast<uint16_t*>(recon);
  const unsigned eb = unsigned((chunks + kFp4Threads - 1) / kFp4Threads);
  if (mx) {                                            // block scales need no stream pass
    if (resid)
      hipLaunchKernelGGL((fp4_encode_kernel<true, true>), dim3(eb), dim3(kFp4Threads), 0, stream, xs, rows, rc, n, T,
                         W, codes, params, tile_start, status);
    else
      hipLaunchKernelGGL((fp4_encode_kernel<false, true>), dim3(eb), dim3(kFp4Threads), 0, stream, xs, rows, rc, n,
                         T, W, codes, params, tile_start, status);
    return hipGetLastError();
  }
  // one partial maximum per amax block, parked in the codes buffer (n*W/2 bytes, room for
  // `chunks` floats), which the encode kernel overwrites after the fold has read it
  const unsigned ab = unsigned(std::min<int64_t>(kAmaxBlocks, (chunks + kFp4Threads - 1) / kFp4Threads));
  float* partial = reinterpret_cast<float*>(codes);
  if (resid) {
    hipLaunchKernelGGL(fp4_amax_kernel<true>, dim3(ab), dim3(kFp4Threads), 0, stream, xs, rows, rc, chunks, W,
                       partial, status);
    hipLaunchKernelGGL(fp4_amax_fold_kernel, dim3(1), dim3(kFp4Threads), 0, stream, partial, int32_t(ab), params);
    hipLaunchKernelGGL((fp4_encode_kernel<true, false>), dim3(eb), dim3(kFp4Threads), 0, stream, xs, rows, rc, n, T,
                       W, codes, params, tile_start, nullptr);
  } else {
    hipLaunchKernelGGL(fp4_amax_kernel<false>, dim3(ab), dim3(kFp4Threads), 0, stream, xs, rows, rc, chunks, W,
                       partial, status);
    hipLaunchKernelGGL(fp4_amax_fold_kernel, dim3(1), dim3(kFp4Threads), 0, stream, partial, int32_t(ab), params);
    hipLaunchKernelGGL((fp4_encode_kernel<false, false>), dim3(eb), dim3(kFp4Threads), 0, stream, xs, rows, rc, n,
                       T, W, codes, params, tile_start, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_fp4_reconstruct(const ChainArgs& chain, bool base_fp4, bool mx, int kind, int32_t T, int32_t H,
                                  int32_t D, void* out, hipStream_t stream) {
  if (D % (mx ? 32 : 16) != 0 || chain.n_loops < 1) return hipErrorInvalidValue;
  const int32_t items = kGroup * (H * D / 16);
  const unsigned parts = unsigned((items + kRecItemsPerThread * kFp4Threads - 1) / (kRecItemsPerThread * kFp4Threads));
  const dim3 grid(unsigned((T + kGroup - 1) / kGroup), parts);
  hipLaunchKernelGGL(fp4_reconstruct_kernel, grid, dim3(kFp4Threads), 0, stream, chain, base_fp4 ? 1 : 0, mx ? 1 : 0,
                     kind, T, H, D, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace flk
