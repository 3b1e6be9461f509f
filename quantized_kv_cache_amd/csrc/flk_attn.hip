// flk_attn.hip -- single-token grouped-query decode attention read straight from packed K/V
// chains (FlashLoop RFC, vllm-rlt #156, section 3.3: optimized readers consume the packed
// base/residual tiles during QK and PV instead of keeping a BF16 shadow cache).
//
// Every wave works alone on a run of 64-token tiles of one KV head, 16 tokens (one MFMA
// slice) at a time, with no block barrier until the end:
//   1. per tile it scatters each compact loop's rows of the tile (found with the tile index)
//      into a wave-private position -> compact-row map, and stages the tile's K parameter rows
//      in wave-private LDS;
//   2. it decodes K_hat of the slice bit for bit as the encoder left it, straight into the A
//      operand registers of S^T = K_hat Q^T (v_mfma_f32_16x16x32_bf16): a lane's A operand is
//      8 consecutive channels of one token, which is exactly one decode item;
//   3. it keeps an online softmax per query head in binary32;
//   4. it decodes V_hat of the slice into a wave-private LDS tile and accumulates
//      O^T += V_hat^T P^T with v_mfma_f32_16x16x16_bf16, whose P^T operand layout is the score
//      tile's register layout, so probabilities never leave registers.
// At the end the block's 4 waves merge their (m, l, O) through LDS into one partial per
// (block, query head); a second kernel merges the partials of all blocks.  A BF16 tail (a
// rolling cache's recent tokens) is read as stored, 16 tokens per wave.
#include <mutex>

#include "flk_device.h"
#include "flk_fp4_device.h"
#include "flk_internal.h"
#include "flk_readers.h"

// The partials buffer of flk_decode_attn_packed_noalloc, for callers that cannot allocate: one
// copy per GPU, held until the process ends, shared by every such call on that GPU.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for the symbol); it uses
// the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[FLK_NOALLOC_SCRATCH_BYTES];

namespace flk {

constexpr int kAThreads = 256;
constexpr int kAttnD = 128;
constexpr int kMaxG = 16;
constexpr int kLdsRow = kAttnD + 8;         // BF16 per LDS row: 272 bytes keep MFMA reads conflict-free
#ifndef FLK_ATTN_WAVES
#define FLK_ATTN_WAVES 8192
#endif
constexpr int kAttnWaves = FLK_ATTN_WAVES;    // aim for about this many waves per launch
#ifndef FLK_ATTN_OCC
#define FLK_ATTN_OCC 2   // waves per SIMD the register budget must allow
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
static int32_t waves_per_head(int32_t tiles, int32_t H) {
  const int32_t cap = kAttnWaves / H > 0 ? kAttnWaves / H : 1;
  return tiles < cap ? (tiles > 0 ? tiles : 1) : cap;
}
static int32_t n_splits(int32_t tiles, int32_t H) { return (waves_per_head(tiles, H) + 3) / 4; }

static int32_t attn_tiles(int32_t T, int32_t tail_len) {
  return (T + kGroup - 1) / kGroup + (tail_len + kGroup - 1) / kGroup;
}

// The workspace a call over T packed tokens and a tail of tail_len tokens uses: one partial
// (m, l, O) per query head and split.
size_t attn_workspace_need(int32_t T, int32_t tail_len, int32_t H, int32_t Hq) {
  return size_t(n_splits(attn_tiles(T, tail_len), H)) * size_t(Hq) * (2 + kAttnD) * sizeof(float);
}

// A bound on attn_workspace_need for every call over at most T_total tokens: such a call has at
// most ceil(T_total/64) + 1 tiles (a packed prefix and a tail may each end in a partial tile),
// and the split count does not decrease with the tile count.
size_t attn_workspace_bytes(int32_t T_total, int32_t H, int32_t Hq) {
  const int64_t tiles = (int64_t(T_total) + kGroup - 1) / kGroup + 1;
  const int32_t s = n_splits(int32_t(tiles < INT32_MAX ? tiles : INT32_MAX), H);
  return size_t(s) * size_t(Hq) * (2 + kAttnD) * sizeof(float);
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

// One wave's LDS: the V_hat slice, the tile's K parameter rows and the compact-row maps.
template <int NL>
struct WaveLds {
  uint16_t v[16][kLdsRow];                 // V_hat of the current slice, [token][channel]
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
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    r.dense[l] = l >= c.n_loops || c.s[l].rows == nullptr;
    r.lo[l] = r.dense[l] ? t0 : uniform(c.s[l].tile_start[tile]);
    r.hi[l] = r.dense[l] ? min(t0 + kGroup, T) : uniform(c.s[l].tile_start[tile + 1]);
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

// Decode 4 items (token tk of the tile, octets oc[i]) of one chain; out[i] receives item i's
// 8 channels as packed BF16 (zeros for an absent or out-of-range token).  Every code word is
// requested first; then one item at a time is decoded, so only one item's binary32 values
// are live.  K: parameters from the staged rows; V: the row's two parameter words, one load.
template <int KIND, int NL, int FMT = 0>
__device__ __forceinline__ void decode_items(const ChainArgs& c, const TileRows<NL>& r, int32_t t0, int32_t T,
                                             int32_t H, int32_t h, int tk, const int oc[4],
                                             const int32_t (*map)[kGroup], const uint32_t (*kp)[2][kAttnD],
                                             const float (&sg)[NL], uint4 out[4]) {
  const int nl = c.n_loops;
  const int32_t t = t0 + tk;
  int32_t j[NL];
  uint32_t cw[NL][4], sw[NL][2];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    j[l] = -1;
    if (l < nl) j[l] = r.dense[l] ? (t < T ? t : -1) : map[l][tk];
    // FP4 loops: the item's block scales in one load -- its 4 E8M0 bytes (MXFP4, one per 32
    // channels) or its 8 E4M3 bytes after the 16-byte header (NVFP4, one per 16 channels);
    // the bytes are picked at decode time, so no load waits before the others are issued
    // (INT4 V loops likewise: the item's two (min, scale) words, one per 64 channels)
    sw[l][0] = sw[l][1] = 0u;
    if ((loop_fp4<FMT>(l) || KIND == FLK_KIND_V) && j[l] >= 0) {
      const uint32_t item = uint32_t(j[l]) * uint32_t(H) + uint32_t(h);
      if (loop_mx<FMT>(l)) {
        sw[l][0] = c.s[l].params[item];
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(c.s[l].params + (loop_nv<FMT>(l) ? 4u : 0u) + item * 2u);
        sw[l][0] = w.x;
        sw[l][1] = w.y;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cw[l][i] = 0;
      if (j[l] >= 0) {
        // uniform base + 32-bit offset: one saddr load, no 64-bit address arithmetic per lane
        const uint32_t item = uint32_t(j[l]) * uint32_t(H) + uint32_t(h);
        cw[l][i] = *reinterpret_cast<const uint32_t*>(c.s[l].codes + (item * (kAttnD / 2) + uint32_t(oc[i]) * 4u));
      }
    }
  }
  // The chain's roundings are taken lazily: acc holds the running sum before its BF16
  // rounding, which happens only when another loop adds to it, or in the final pack.  The
  // result is the encoder's bf16(...bf16(bf16(base) + bf16(d2)) ... + bf16(dR)).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (j[l] < 0) continue;
      float d[8];
      if (loop_fp4<FMT>(l)) {          // octet oc's block: byte oc / 4 (MXFP4) or oc / 2 (NVFP4)
        const uint32_t b = loop_mx<FMT>(l) ? uint32_t(oc[i]) >> 2 : uint32_t(oc[i]) >> 1;
        const uint32_t sb = (((b & 4u) ? sw[l][1] : sw[l][0]) >> (8u * (b & 3u))) & 0xFFu;
        fp4_decode8(cw[l][i], loop_mx<FMT>(l) ? fp4_e8m0_value(sb) : fp4_e4m3_value(sb) * sg[l], d);
      } else {
        uint32_t p[8];
        if (KIND == FLK_KIND_K) {
          const int rg = c.ktile ? 0 : (j[l] / kGroup) & 1;  // staged by rowgroup parity
          const uint4 a = *reinterpret_cast<const uint4*>(&kp[l][rg][oc[i] * 8]);
          const uint4 b = *reinterpret_cast<const uint4*>(&kp[l][rg][oc[i] * 8 + 4]);
          p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w; p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
        } else {                                         // V: the octet's 64-channel group
          const uint32_t w = (oc[i] >> 3) ? sw[l][1] : sw[l][0];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = w;
        }
        decode_item(cw[l][i], p, d);
      }
      if (l == 0) {                                      // the dense base: every live token
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = d[e];
      } else {
        round_bf16x8_inplace(acc);
        round_bf16x8_inplace(d);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + d[e];
      }
    }
    out[i] = round_bf16x8(acc);                          // RNE pack of the last sum
  }
}

// SC: also write every (query head, packed token) scaled score to scores[head][position], rows
// of ceil(T/4)*4 floats (the reference loop of sparse decode attention selects keys from them).
template <int NL, bool SC, int FMT = 0>
__global__ __launch_bounds__(kAThreads, FLK_ATTN_OCC) void attn_wave_kernel(ChainArgs kc, ChainArgs vc, int32_t T, int32_t H,
                                                              int32_t G, const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ kt,
                                                              const uint16_t* __restrict__ vt, int32_t tail_len,
                                                              float scale, int32_t wph,
                                                              float* __restrict__ ws_ml, float* __restrict__ ws_o,
                                                              float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[attn_lds_bytes<NL>()];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;                                // MFMA column: query head / token / channel
  const int kb = lane >> 4;                               // MFMA k-block / row block
  // Blocks are renumbered split-major, head-minor, and each XCD runs a contiguous range of the
  // new numbers: the H heads of a token range run together in one L2.  A token's codes of heads
  // 2m and 2m+1 share a 128-byte line, and a row's V parameters of all heads share one, so
  // those lines are fetched once instead of once per head.
  const uint32_t lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int32_t split = int32_t(lin / gridDim.y);
  const int32_t h = int32_t(lin % gridDim.y);
  const int32_t Hq = H * G;
  const int32_t ptiles = (T + kGroup - 1) / kGroup;       // packed tiles
  // the head's packed tiles, ptiles / wph per wave and one more for the first ptiles % wph
  const int32_t w = split * kAWaves + wave;               // this wave's index within its head
  const int32_t base = ptiles / wph, extra = ptiles - base * wph;
  const int32_t tile0 = w < wph ? w * base + min(w, extra) : ptiles;
  const int32_t tile1 = w < wph ? tile0 + base + (w < extra ? 1 : 0) : ptiles;
  WaveLds<NL>& L = reinterpret_cast<WaveLds<NL>*>(s_raw)[wave];

  // Q^T as the B operand of S^T = K_hat Q^T: lane holds Q[n][32*ks + 8*kb + j], zero past G
  bf16x8_t qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < G) w = *reinterpret_cast<const uint4*>(q + int64_t(h * G + n) * kAttnD + 32 * ks + 8 * kb);
    qb[ks] = __builtin_bit_cast(bf16x8_t, w);
  }
  // decode items of this lane: token n of the slice, octets 4*i + kb (the K A-operand layout)
  int oc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oc[i] = 4 * i + kb;

  // NVFP4 loops: the stream scales, loaded once (kept out of the tile loop, where their scalar
  // loads would share a wait counter with the LDS reads of the K parameter rows)
  float sgk[NL], sgv[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    sgk[l] = loop_nv<FMT>(l) && l < kc.n_loops ? __uint_as_float(kc.s[l].params[0]) : 0.0f;
    sgv[l] = loop_nv<FMT>(l) && l < vc.n_loops ? __uint_as_float(vc.s[l].params[0]) : 0.0f;
  }

  float m_run = -__builtin_inff(), l_run = 0.0f;
  float4_t o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // One 16-token slice: S^T = K Q^T on the MFMA, the online softmax, then V (from load_v,
  // called after the softmax so one operand set is live at a time) into LDS and
  // O^T += V^T P^T.  Slots 16*sl + 4*kb + i at or past n_valid are masked.
  auto attend_slice = [&](const uint4 (&kitem)[4], int sl, int32_t n_valid, auto&& load_v, auto&& emit) {
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kitem[ks]), qb[ks], sacc, 0, 0, 0);
    // online softmax; lane holds the scores of tokens 4*kb + i of the slice for head n
    float sc[4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = 16 * sl + 4 * kb + i < n_valid ? sacc[i] * scale : -__builtin_inff();
      mx = fmaxf(mx, sc[i]);
    }
    emit(sc);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float p[4], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = m_new == -__builtin_inff() ? 0.0f : __expf(sc[i] - m_new);
      psum += p[i];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    const float corr = m_run == -__builtin_inff() ? 0.0f : __expf(m_run - m_new);
    l_run = l_run * corr + psum;
    m_run = m_new;

    uint4 vitem[4];
    load_v(vitem);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&L.v[n][oc[i] * 8]) = vitem[i];
    wave_sync();
    short4_t pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) pb[j] = short(__builtin_bit_cast(uint16_t, (__bf16)p[j]));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      short4_t a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = short(L.v[4 * kb + j][16 * mt + n]);
      o[mt] = o[mt] * corr;
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[mt], 0, 0, 0);
    }
    wave_sync();                                          // the slice's V reads before the next writes
  };

  // The BF16 tail, read as stored, in 16-token slices: slice s goes to waves s, s + wph, ...
  // of every head, a small addition to many waves rather than whole tiles for a few.
  const int32_t tail_slices = (tail_len + 15) / 16;
  for (int32_t ts = w; w < wph && ts < tail_slices; ts += wph) {
    const int32_t n_valid = min(16, tail_len - 16 * ts);
    const bool ok = n < n_valid;
    const int64_t base = (int64_t(16 * ts + n) * H + h) * kAttnD;
    uint4 item[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      item[i] = ok ? *reinterpret_cast<const uint4*>(kt + base + oc[i] * 8) : make_uint4(0, 0, 0, 0);
    attend_slice(item, 0, n_valid, [&](uint4 (&v)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = ok ? *reinterpret_cast<const uint4*>(vt + base + oc[i] * 8) : make_uint4(0, 0, 0, 0);
    }, [](const float (&)[4]) {});
  }

  for (int32_t tile = tile0; tile < tile1; ++tile) {
    const int32_t t0 = tile * kGroup;
    const TileRows<NL> rk = tile_rows<NL>(kc, tile, T);
    const TileRows<NL> rv = tile_rows<NL>(vc, tile, T);
    wave_sync();                                          // the previous tile's LDS reads are done
    build_maps<NL>(kc, rk, t0, L.map[0], lane);
    build_maps<NL>(vc, rv, t0, L.map[1], lane);
    // K parameter rows of the tile: rowgroup lo/64 (and lo/64 + 1 for a compact loop), each in
    // the slot of its parity, so a row j finds its parameters in slot (j/64) & 1; with tile
    // groups, the tile's own row in slot 0
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (l >= kc.n_loops || loop_fp4<FMT>(l)) continue;    // FP4 loops carry no K parameter rows
      if (kc.ktile) {
        if (rk.hi[l] > rk.lo[l]) {
          const uint2 w = *reinterpret_cast<const uint2*>(kc.s[l].params + (uint32_t(tile) * uint32_t(H) + uint32_t(h)) * kAttnD + 2 * lane);
          *reinterpret_cast<uint2*>(&L.kp[l][0][2 * lane]) = w;
        }
        continue;
      }
      const int32_t nrg = (kc.s[l].n + kGroup - 1) / kGroup;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int32_t rg = rk.lo[l] / kGroup + r;
        if ((r == 1 && rk.dense[l]) || rg >= nrg) continue;
        const uint2 w = *reinterpret_cast<const uint2*>(kc.s[l].params + (uint32_t(rg) * uint32_t(H) + uint32_t(h)) * kAttnD + 2 * lane);
        *reinterpret_cast<uint2*>(&L.kp[l][rg & 1][2 * lane]) = w;
      }
    }
    // Order the tile's positions so that positions listed by the same loops sit together (the
    // softmax sum does not depend on the order): a 16-token slice then mostly holds one loop
    // pattern, and a loop none of its tokens has is skipped by the whole wave.  Positions past
    // T go last.  Groups are ranked in order of first occurrence.
    const int32_t n_valid = min(kGroup, T - t0);
    {
      uint32_t key = 0;
#pragma unroll
      for (int l = 1; l < NL; ++l) {
        if (l < kc.n_loops && !rk.dense[l] && L.map[0][l][lane] >= 0) key |= 1u << l;
        if (l < vc.n_loops && !rv.dense[l] && L.map[1][l][lane] >= 0) key |= 1u << (NL + l);
      }
      const bool valid = lane < n_valid;
      const uint64_t below = (uint64_t(1) << lane) - 1;
      uint64_t remaining = __ballot(valid);
      int base = 0, rank = 0;
      while (remaining) {
        const int leader = __builtin_ctzll(remaining);
        const uint32_t k = __builtin_amdgcn_readlane(key, leader);
        const uint64_t grp = __ballot(valid && key == k);
        if (valid && key == k) rank = base + __builtin_popcountll(grp & below);
        base += __builtin_popcountll(grp);
        remaining &= ~grp;
      }
      if (!valid) rank = lane;                              // the invalid tail keeps its order
      L.perm[rank] = lane;
    }
    wave_sync();

    for (int sl = 0; sl < kGroup / 16; ++sl) {
      const int tk = L.perm[16 * sl + n];
      // K_hat of the slice straight into the A operands
      uint4 item[4];
      decode_items<FLK_KIND_K, NL, FMT>(kc, rk, t0, T, H, h, tk, oc, L.map[0], L.kp, sgk, item);
      attend_slice(item, sl, n_valid, [&](uint4 (&v)[4]) {
        decode_items<FLK_KIND_V, NL, FMT>(vc, rv, t0, T, H, h, tk, oc, L.map[1], L.kp, sgv, v);
      }, [&](const float (&sc)[4]) {
        if constexpr (SC) {
          if (n < G) {
            float* row = scores + int64_t(h * G + n) * ((int64_t(T) + 3) & ~int64_t(3)) + t0;  // rows padded to 16 B
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int slot = 16 * sl + 4 * kb + i;
              if (slot < n_valid) row[L.perm[slot]] = sc[i];
            }
          }
        }
      });
    }
  }

  // merge the 4 waves: (m, l) per head and O^T per (head, channel) through LDS
  __syncthreads();
  float* s_m = reinterpret_cast<float*>(s_raw);           // [4][16]
  float* s_l = s_m + kAWaves * kMaxG;                     // [4][16]
  float* s_o = s_l + kAWaves * kMaxG;                     // [4][16][128]
  if (kb == 0) {
    s_m[wave * kMaxG + n] = m_run;
    s_l[wave * kMaxG + n] = l_run;
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[(wave * kMaxG + n) * kAttnD + 16 * mt + 4 * kb + i] = o[mt][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kAttnD; idx += kAThreads) {
    const int g = idx / kAttnD, ch = idx % kAttnD;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAWaves; ++w) M = fmaxf(M, s_m[w * kMaxG + g]);
    float Ls = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kAWaves; ++w) {
      const float mw = s_m[w * kMaxG + g];
      const float f = mw == -__builtin_inff() ? 0.0f : __expf(mw - M);
      Ls += s_l[w * kMaxG + g] * f;
      O += s_o[(w * kMaxG + g) * kAttnD + ch] * f;
    }
    const int64_t qi = int64_t(split) * Hq + h * G + g;
    if (ch == 0) { ws_ml[2 * qi] = M; ws_ml[2 * qi + 1] = Ls; }
    ws_o[qi * kAttnD + ch] = O;
  }
}

// Merge the per-block partials of one query head (blockIdx.x).  Thread (c = tid % 128,
// g = tid / 128) takes channel c of every kCombGroups-th split from g on, with independent
// loads in flight; the groups then merge through LDS.
constexpr int kCombGroups = 8;
__global__ __launch_bounds__(kAttnD * kCombGroups) void attn_combine_kernel(int32_t splits, int32_t Hq,
                                                                            const float* __restrict__ ws_ml,
                                                                            const float* __restrict__ ws_o,
                                                                            uint16_t* __restrict__ out,
                                                                            float* __restrict__ out32,
                                                                            float* __restrict__ ml_out) {
  __shared__ float s_red[kCombGroups * kAttnD];
  __shared__ float s_l[kCombGroups * kAttnD];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid % kAttnD, g = tid / kAttnD;
  // global maximum of the partial maxima
  float M = -__builtin_inff();
  for (int s = tid; s < splits; s += kAttnD * kCombGroups) M = fmaxf(M, ws_ml[2 * (int64_t(s) * Hq + i)]);
  s_red[tid] = M;
  __syncthreads();
  for (int w = kAttnD * kCombGroups / 2; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
    __syncthreads();
  }
  M = s_red[0];
  __syncthreads();
  float L = 0.0f, O = 0.0f;
#pragma unroll 8
  for (int s = g; s < splits; s += kCombGroups) {
    const int64_t qi = int64_t(s) * Hq + i;
    const float m = ws_ml[2 * qi];
    const float w = m == -__builtin_inff() ? 0.0f : __expf(m - M);
    L = __builtin_fmaf(ws_ml[2 * qi + 1], w, L);
    O = __builtin_fmaf(ws_o[qi * kAttnD + c], w, O);
  }
  s_red[tid] = O;
  s_l[tid] = L;
  __syncthreads();
  if (g == 0) {
    float Ot = 0.0f, Lt = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombGroups; ++k) {
      Ot += s_red[k * kAttnD + c];
      Lt += s_l[k * kAttnD + c];
    }
    out[int64_t(i) * kAttnD + c] = __builtin_bit_cast(uint16_t, (__bf16)(Ot / Lt));
    if (out32) out32[int64_t(i) * kAttnD + c] = Ot / Lt;     // the sparse reference's O_ref
    if (ml_out && c == 0) {                                   // and its softmax max and denominator
      ml_out[2 * i] = M;
      ml_out[2 * i + 1] = Lt;
    }
  }
}

template <bool SC, int FMT = 0>
static hipError_t launch_attn(int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                              const ChainArgs& vc, const void* k_tail, const void* v_tail, int32_t tail_len,
                              float scale, void* out, float* out32, float* ml_out, float* scores, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (ws == nullptr || ws_bytes < attn_workspace_need(T, tail_len, H, Hq)) return hipErrorInvalidValue;
  const int32_t tiles = attn_tiles(T, tail_len);
  const int32_t wph = waves_per_head(tiles, H);
  const int32_t splits = n_splits(tiles, H);
  const int32_t G = Hq / H;
  float* ws_ml = static_cast<float*>(ws);
  float* ws_o = ws_ml + size_t(splits) * Hq * 2;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* ktp = static_cast<const uint16_t*>(k_tail);
  const uint16_t* vtp = static_cast<const uint16_t*>(v_tail);
  int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  if (nl < 1) nl = 1;                              // no packed tokens: only the tail's tiles run
  const dim3 grid(static_cast<unsigned>(splits), static_cast<unsigned>(H));
#define FLK_A(NLV)                                                                                          \
  case NLV:                                                                                                 \
    hipLaunchKernelGGL((attn_wave_kernel<NLV, SC, FMT>), grid, dim3(kAThreads), 0, stream, kc, vc, T, H, G, qp, \
                       ktp, vtp, tail_len, scale, wph, ws_ml, ws_o, scores);                                \
    break;
  switch (nl) {
    FLK_A(1) FLK_A(2) FLK_A(3) FLK_A(4) FLK_A(5) FLK_A(6) FLK_A(7) FLK_A(8)
    default: return hipErrorInvalidValue;
  }
#undef FLK_A
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(Hq), dim3(kAttnD * kCombGroups), 0, stream, splits, Hq, ws_ml,
                     ws_o, static_cast<uint16_t*>(out), out32, ml_out);
  return hipGetLastError();
}

hipError_t launch_decode_attn(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, const void* k_tail,
                              const void* v_tail, int32_t tail_len, float scale, void* out,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)D;
  return launch_attn<false>(T, H, Hq, q, kc, vc, k_tail, v_tail, tail_len, scale, out, nullptr, nullptr, nullptr,
                            ws, ws_bytes, stream);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];    // device address of `scratch` per device, found once

// The current device's copy of `scratch`, looked up on the first call on that device.
hipError_t scratch_address(void** p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *p = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_decode_attn_noalloc(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q, const ChainArgs& kc,
                                      const ChainArgs& vc, float scale, void* out, hipStream_t stream) {
  if (attn_workspace_need(T, 0, H, Hq) > size_t(FLK_NOALLOC_SCRATCH_BYTES)) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  // every partial the combine reads is written by the attention kernel first: nothing to clear
  return launch_decode_attn(T, H, D, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, ws,
                            size_t(FLK_NOALLOC_SCRATCH_BYTES), stream);
}

hipError_t launch_decode_attn_fmt(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                                  const ChainArgs& vc, float scale, void* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  switch (fmt) {
    case 0:
      return launch_attn<false, 0>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 1:
      return launch_attn<false, 1>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 2:
      return launch_attn<false, 2>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 3:
      return launch_attn<false, 3>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 4:
      return launch_attn<false, 4>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_reference(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                                 const ChainArgs& vc, float scale, void* out, float* o_ref, float* ml,
                                 float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
#define FLK_R(F)                                                                                                  \
  case F:                                                                                                         \
    return launch_attn<true, F>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, o_ref, ml, scores, ws,      \
                                ws_bytes, stream);
  switch (fmt) {
    FLK_R(0) FLK_R(1) FLK_R(2) FLK_R(3) FLK_R(4)
    default: return hipErrorInvalidValue;
  }
#undef FLK_R
}

}  // namespace flk
