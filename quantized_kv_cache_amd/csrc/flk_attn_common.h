// flk_attn_common.h -- pieces shared by the decode-attention kernels that read packed chains:
// the wave and split partition of the tokens, the per-tile compact-row maps and K parameter
// staging, the exact decode of K_hat / V_hat items into MFMA operands, and the helpers of the
// PV products taken straight from INT4 codes.
#pragma once

#include "flk_device.h"
#include "flk_fp4_device.h"
#include "flk_internal.h"
#include "flk_readers.h"

namespace flk {

constexpr int kAThreads = 256;
constexpr int kAttnD = 128;
constexpr int kMaxG = 16;
constexpr int kLdsRow = kAttnD + 8;         // BF16 per LDS row: 272 bytes keep MFMA reads conflict-free
#ifndef FLK_ATTN_WAVES
#define FLK_ATTN_WAVES 8192
#endif
constexpr int kAttnWaves = FLK_ATTN_WAVES;    // aim for about this many waves per launch
// The two-pass reader's launches: one round of 4 waves per SIMD on 256 CUs (4096 waves) beats
// two rounds (8192) by about 3 %; the one-pass reader keeps 8192 (4096 is 6 % slower there).
#ifndef FLK_SPLIT_ATTN_WAVES
#define FLK_SPLIT_ATTN_WAVES 4096
#endif
constexpr int kSplitAttnWaves = FLK_SPLIT_ATTN_WAVES;
constexpr int kSplitFp4Loops = 4;          // FP4 chains up to this depth take the two-pass reader
#ifndef FLK_ATTN_OCC
#define FLK_ATTN_OCC 3   // waves per SIMD the register budget must allow
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Waves per KV head: about kAttnWaves waves per launch, never more than one per tile.  The
// waves of a head share its tiles with counts that differ by at most one (the first waves take
// the extra ones), so a few extra tiles (a BF16 tail) lengthen a few early waves instead of
// adding blocks.  A block
// of 4 waves writes one partial per query head.  `tiles` counts the packed tiles and the
// tiles of a BF16 tail together.
inline int32_t waves_per_head(int32_t tiles, int32_t H, int32_t waves = kAttnWaves) {
  const int32_t cap = waves / H > 0 ? waves / H : 1;
  return tiles < cap ? (tiles > 0 ? tiles : 1) : cap;
}
inline int32_t n_splits(int32_t tiles, int32_t H, int32_t waves = kAttnWaves) {
  return (waves_per_head(tiles, H, waves) + 3) / 4;
}
static_assert(kSplitAttnWaves <= kAttnWaves, "workspace sizes count the larger split count");

inline int32_t attn_tiles(int32_t T, int32_t tail_len) {
  return (T + kGroup - 1) / kGroup + (tail_len + kGroup - 1) / kGroup;
}

// Decode loop l's 8 channels of one item into d[], the binary32 values min + scale * code
// before their BF16 rounding (the caller rounds them where the chain needs it).  K: params of
// the 8 channels come from the LDS copy of the item's parameter row; V: one parameter for the
// item's 64-channel group.
__device__ __forceinline__ void decode_item(uint32_t cw, const uint32_t p[8], float d[8]) {
  float c[8];
  codes8_to_f32(cw, c);
#pragma unroll
  for (int e = 0; e < 8; ++e) d[e] = decode(c[e], f16_bits_to_f32(p[e] & 0xFFFFu), f16_bits_to_f32(p[e] >> 16));
}


__device__ __forceinline__ void store_bf16x8(uint16_t* dst, const float v[8]) {
  *reinterpret_cast<uint4*>(dst) = pack_exact_bf16x8(v);
}
__device__ __forceinline__ void load_bf16x8(const uint16_t* src, float v[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(src);
  v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xFFFF0000u);
  v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xFFFF0000u);
  v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xFFFF0000u);
  v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xFFFF0000u);
}

constexpr int kAWaves = kAThreads / 64;

// One wave's LDS: the V slice (decoded V_hat, or the INT4 codes and parameters as loaded),
// the tile's K parameter rows and the compact-row maps.
template <int NL>
struct WaveLds {
  union {
    uint16_t v[16][kLdsRow];               // V_hat of the current slice, [token][channel]
    struct {
      uint8_t codes[NL][16][kAttnD / 2];   // per loop: the slice's 16 code rows (16-byte chunks
                                           // of row r at chunk q ^ (r / 4 % 4), see vchunk)
      uint32_t params[NL][64];             // per loop: rows 0..15 x (group 0, group 1) words
    } vs;
  };
  uint32_t kp[NL][2][kAttnD];              // K parameter rows of the tile (two rowgroups)
  int32_t map[2][NL][kGroup];              // [K|V][loop][position in tile] -> compact row, -1 absent
  int32_t perm[kGroup];                    // tile positions grouped by which loops list them
};
constexpr size_t kMergeBytes = size_t(kAWaves) * kMaxG * (2 + kAttnD) * sizeof(float);
template <int NL>
constexpr size_t attn_lds_bytes() {
  return kAWaves * sizeof(WaveLds<NL>) > kMergeBytes ? kAWaves * sizeof(WaveLds<NL>) : kMergeBytes;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per chain and loop: the rows of the tile [lo, hi) and whether the loop is dense.
template <int NL>
struct TileRows {
  int32_t lo[NL], hi[NL];
  bool dense[NL];
};

template <int NL>
__device__ __forceinline__ TileRows<NL> tile_rows(const ChainArgs& c, int32_t tile, int32_t T) {
  TileRows<NL> r;
  const int32_t t0 = tile * kGroup;
  // every loop's pair of tile-index entries is requested before any is used: one round trip
  int2 e[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    r.dense[l] = l >= c.n_loops || c.s[l].rows == nullptr;
    e[l] = make_int2(t0, min(t0 + kGroup, T));
    if (!r.dense[l]) e[l] = make_int2(c.s[l].tile_start[tile], c.s[l].tile_start[tile + 1]);
  }
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    r.lo[l] = uniform(e[l].x);
    r.hi[l] = uniform(e[l].y);
  }
  return r;
}

// Scatter the tile's compact rows of every compact loop into map[l][position - t0].
template <int NL>
__device__ __forceinline__ void build_maps(const ChainArgs& c, const TileRows<NL>& r, int32_t t0,
                                           int32_t (*map)[kGroup], int lane) {
#pragma unroll
  for (int l = 0; l < NL; ++l)
    if (l < c.n_loops && !r.dense[l]) map[l][lane] = -1;
  wave_sync();
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (l >= c.n_loops || r.dense[l]) continue;
    const int32_t j = r.lo[l] + lane;
    if (j < r.hi[l]) {
      const uint32_t p = uint32_t(c.s[l].rows[j] - t0);
      if (p < uint32_t(kGroup)) map[l][p] = j;         // a malformed entry outside the tile is dropped
    }
  }
}

// The loads of one item set (token tk of a tile, octets oc[]) of one chain: each loop's compact
// row (-1 when the loop does not list the token), code words and, for FP4 and V loops, the scale
// words.  issue_items requests them; decode_loaded turns them into K_hat / V_hat.
template <int NL>
struct ItemLoads {
  int32_t j[NL];
  uint32_t cw[NL][4], sw[NL][2];
};

template <int KIND, int NL, int FMT = 0>
__device__ __forceinline__ void issue_items(const ChainArgs& c, const TileRows<NL>& r, int32_t t0, int32_t T,
                                            int32_t H, int32_t h, int tk, const int oc[4],
                                            const int32_t (*map)[kGroup], ItemLoads<NL>& ld) {
  const int nl = c.n_loops;
  const int32_t t = t0 + tk;
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    ld.j[l] = -1;
    if (l < nl) ld.j[l] = r.dense[l] ? (t < T ? t : -1) : map[l][tk];
    // FP4 loops: the item's block scales in one load -- its 4 E8M0 bytes (MXFP4, one per 32
    // channels) or its 8 E4M3 bytes after the 16-byte header (NVFP4, one per 16 channels);
    // the bytes are picked at decode time, so no load waits before the others are issued
    // (INT4 V loops likewise: the item's two (min, scale) words, one per 64 channels)
    ld.sw[l][0] = ld.sw[l][1] = 0u;
    if ((loop_fp4<FMT>(l) || KIND == FLK_KIND_V) && ld.j[l] >= 0) {
      const uint32_t item = uint32_t(ld.j[l]) * uint32_t(H) + uint32_t(h);
      if (loop_mx<FMT>(l)) {
        ld.sw[l][0] = c.s[l].params[item];
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(c.s[l].params + (loop_nv<FMT>(l) ? 4u : 0u) + item * 2u);
        ld.sw[l][0] = w.x;
        ld.sw[l][1] = w.y;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ld.cw[l][i] = 0;
      if (ld.j[l] >= 0) {
        // uniform base + 32-bit offset: one saddr load, no 64-bit address arithmetic per lane
        const uint32_t item = uint32_t(ld.j[l]) * uint32_t(H) + uint32_t(h);
        ld.cw[l][i] = *reinterpret_cast<const uint32_t*>(c.s[l].codes + (item * (kAttnD / 2) + uint32_t(oc[i]) * 4u));
      }
    }
  }
}

template <int KIND, int NL, int FMT = 0>
__device__ __forceinline__ void decode_loaded(const ChainArgs& c, const ItemLoads<NL>& ld, const int oc[4],
                                              const uint32_t (*kp)[2][kAttnD], const float (&sg)[NL],
                                              uint4 out[4]) {
  // The chain's roundings are taken lazily: acc holds the running sum before its BF16
  // rounding, which happens only when another loop adds to it, or in the final pack.  The
  // result is the encoder's bf16(...bf16(bf16(base) + bf16(d2)) ... + bf16(dR)).
  const uint32_t ones = bf16_ones();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (ld.j[l] < 0) continue;
      float d[8];
      if (loop_fp4<FMT>(l)) {          // octet oc's block: byte oc / 4 (MXFP4) or oc / 2 (NVFP4)
        const uint32_t b = loop_mx<FMT>(l) ? uint32_t(oc[i]) >> 2 : uint32_t(oc[i]) >> 1;
        const uint32_t sb = (((b & 4u) ? ld.sw[l][1] : ld.sw[l][0]) >> (8u * (b & 3u))) & 0xFFu;
        fp4_decode8(ld.cw[l][i], loop_mx<FMT>(l) ? fp4_e8m0_value(sb) : fp4_e4m3_value(sb) * sg[l], d);
      } else {
        uint32_t p[8];
        if (KIND == FLK_KIND_K) {
          const int rg = c.ktile ? 0 : (ld.j[l] / kGroup) & 1;  // staged by rowgroup parity
          const uint4 a = *reinterpret_cast<const uint4*>(&kp[l][rg][oc[i] * 8]);
          const uint4 b = *reinterpret_cast<const uint4*>(&kp[l][rg][oc[i] * 8 + 4]);
          p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w; p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
        } else {                                         // V: the octet's 64-channel group
          const uint32_t w = (oc[i] >> 3) ? ld.sw[l][1] : ld.sw[l][0];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = w;
        }
        decode_item(ld.cw[l][i], p, d);
      }
      if (l == 0) {                                      // the dense base: every live token
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = d[e];
      } else {
        add_rounded_bf16x8(acc, d, ones);
      }
    }
    out[i] = round_bf16x8(acc);                          // RNE pack of the last sum
  }
}

// Decode 4 items (token tk of the tile, octets oc[i]) of one chain; out[i] receives item i's
// 8 channels as packed BF16 (zeros for an absent or out-of-range token).  Every code word is
// requested first; then one item at a time is decoded, so only one item's binary32 values
// are live.  K: parameters from the staged rows; V: the row's two parameter words, one load.
template <int KIND, int NL, int FMT = 0>
__device__ __forceinline__ void decode_items(const ChainArgs& c, const TileRows<NL>& r, int32_t t0, int32_t T,
                                             int32_t H, int32_t h, int tk, const int oc[4],
                                             const int32_t (*map)[kGroup], const uint32_t (*kp)[2][kAttnD],
                                             const float (&sg)[NL], uint4 out[4]) {
  ItemLoads<NL> ld;
  issue_items<KIND, NL, FMT>(c, r, t0, T, H, h, tk, oc, map, ld);
  decode_loaded<KIND, NL, FMT>(c, ld, oc, kp, sg, out);
}

// ---- the PV products ---------------------------------------------------------------------------
// O^T += V^T P^T runs on 16x16x16 MFMAs: M = 16 channels per output tile (8 tiles for D = 128),
// N = the query heads, K = the 16 tokens of a slice.  Output tile mt, row m holds channel
// pv_channel(mt, m): tiles 0-3 the 64 channels of V group 0, tiles 4-7 those of group 1, and
// row m of a group's four tiles the channels 4m .. 4m+3.  In that order the channels of row m
// are exactly the nibbles of a token's code bytes 2m, 2m+1 (group 0) and 32+2m, 33+2m (group 1):
// nibble k of the word those two 16-bit halves form belongs to tile k.
__device__ __forceinline__ constexpr int pv_channel(int mt, int m) { return 64 * (mt >> 2) + 4 * m + (mt & 3); }

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};           // v_cvt_pk_f16_f32, nearest-even
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f16x4_t f16x4_of(uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t w = {lo, hi};
  return __builtin_bit_cast(f16x4_t, w);
}
__device__ __forceinline__ uint32_t buf_ld16(BufRsrc r, uint32_t voff) {
  return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, int(voff), 0, 0));
}
__device__ __forceinline__ uint2 buf_ld64(BufRsrc r, uint32_t voff) {
  typedef uint32_t v2 __attribute__((ext_vector_type(2)));
  const v2 v = __builtin_amdgcn_raw_buffer_load_b64(r, int(voff), 0, 0);
  return make_uint2(v.x, v.y);
}
constexpr uint32_t kOutOfRange = 0xFFFFFF00u;   // a lane offset past any stream: the load reads 0

// The staged code rows of a slice: a row's four 16-byte chunks are stored XOR-swizzled by the
// row's quarter of the slice, so that the four k-blocks' 16-bit reads of one byte column fall in
// different LDS banks.
__device__ __forceinline__ int vchunk(int row, int q) { return q ^ ((row >> 2) & 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The same address, opaque to the optimizer: loads through it are not hoisted out of the loop
// they sit in, so the values they read are not held in registers across the whole kernel.
template <typename T>
__device__ __forceinline__ const T* opaque_ptr(const T* p) {
  asm volatile("" : "+s"(p));
  return p;
}


// The two-pass decode attention over INT4 chains and an optional BF16 tail (flk_attn_split.hip):
// scores (binary32 rows of ceil((T + tail_len)/4)*4 per query head, the tail's after the packed
// positions) and block maxima, then the PV partials (m, l, O) per split and query head that
// attn_combine_kernel merges.
hipError_t launch_attn_split(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                             const ChainArgs& vc, const void* k_tail, const void* v_tail, int32_t tail_len,
                             float scale, int32_t wph, int32_t splits, float* scores, float* block_max, float* ws_ml,
                             float* ws_o, hipStream_t stream);

}  // namespace flk
