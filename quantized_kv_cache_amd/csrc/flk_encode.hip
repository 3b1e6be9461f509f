// flk_encode.hip -- gfx950 encode kernels: quantized base and cross-loop residuals.
//
// One pass per loop: each block loads its tile of X[r] (and, for a residual, the gathered
// rows of X_hat[r-1]) once with 16-byte loads, forms the BF16 residual in registers,
// reduces group extremes, derives FP16 params, writes nibble-packed codes and params, and
// writes the updated reconstruction back in place.  The method is the FlashLoop RFC
// (vllm-rlt #156) section 3.3; group axes and storage follow vllm-rlt PR #166 "Purpose".
#include <type_traits>

#include "flk_device.h"
#include "flk_internal.h"

namespace flk {

constexpr int kThreads = 256;
#ifndef FLK_VWIDE_WAVES
#define FLK_VWIDE_WAVES 32768
#endif
constexpr int kVWideWaves = FLK_VWIDE_WAVES;
// K block width: compact loops run one or two rounds of blocks, so they take narrower blocks
// (twice as many, 2 rows per thread) to overlap their load-reduce-store chains; base and dense
// loops keep 128 channels.
template <bool SPARSE>
constexpr int k_block_channels() { return SPARSE ? 64 : 128; }

constexpr uint32_t kDevRows = FLK_DEV_ROWS;

__device__ __forceinline__ void unpack8(const uint4& w, float v[8]) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

__device__ __forceinline__ uint4 pack8(const float v[8]) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  return w;
}

// First index of the ascending rows[0..n) whose value is >= key, found by one wave in rounds
// of 64 parallel probes (ceil(log64(n)) dependent loads).  Every lane returns the same value;
// call with the whole wave active.
__device__ __forceinline__ int32_t wave_lower_bound(const int32_t* __restrict__ rows, int32_t n, int32_t key,
                                                    int lane) {
  int32_t a = 0, b = n;                    // the answer lies in [a, b]
  while (a < b) {
    const int32_t s = (b - a + 63) / 64;
    const int32_t idx = a + lane * s;
    const bool pred = idx < b && rows[idx] < key;
    const int32_t c = __builtin_popcountll(__ballot(pred));
    if (c == 0) return a;
    const int32_t na = a + (c - 1) * s + 1;
    const int32_t nb = min(a + c * s, b);
    if (s == 1) return nb;
    a = na;
    b = nb;
  }
  return a;
}

// Compact loops of at most this many rows (a rolling-tail flush, a short request) find each
// tile's rows with an in-wave search and write the tile index themselves; longer ones read
// the index that tile_index_kernel writes first (one load instead of a search in front of
// every wave's data loads).
constexpr int32_t kTileSearchRows = 4096;

// ---------------------------------------------------------------------------------------
// K, tile (page-local) groups, compact loops: a wave owns the compact rows of one
// 64-position tile (0 to 64 of them) for 64 channels, and the 4 waves of a block take
// neighbouring channel strips.  Lane (rs, cc) = (lane >> 3, lane & 7) holds 8 channels of
// octet cc for rows rs, rs + 8, ... of the tile: 8 consecutive lanes cover one row's 128
// bytes, so every load and store merges like a row-major access.  A group's extremes take
// a reduce-scatter across the row-slot lanes (two cross-row shuffles and a DPP rotation,
// halving the channels each step) -- no LDS, no barrier -- after which each lane derives
// and writes the params of one channel of its octet (one 256-byte store per wave) and the
// octet exchanges them.  A tile holds few rows
// at low retention, so many independent short waves hide the load latency better than a
// block reduction would.  The tile's row range comes from the tile index, which
// tile_index_kernel writes first (a search per wave would put several dependent loads in
// front of every wave's data loads).
// ---------------------------------------------------------------------------------------
template <bool RESID>
__device__ __forceinline__ void encode_k_tile_body(const EncArgs& a, uint32_t item) {
  const int32_t* __restrict__ rows = a.rows;
  uint16_t* __restrict__ recon = a.recon;
  const int32_t n = a.n, T = a.T, W = a.W, pos0 = a.pos0;
  const int lane = threadIdx.x & 63;
  const uint32_t nstrips = (uint32_t(W >> 3) + 7u) / 8u;
  const int32_t tile = int32_t(item / nstrips);
  const uint32_t strip = item - uint32_t(tile) * nstrips;
  if (tile >= (T + kGroup - 1) / kGroup) return;          // wave-uniform
  const int cc = lane & 7, rs = lane >> 3;
  const int32_t chunk = int32_t(strip) * 8 + cc;
  const bool cact = chunk < (W >> 3);
  const int64_t ch = int64_t(chunk) * 8;

  // the tile's compact rows [jbeg, jend): searched in rows for a short loop, else from the tile
  // index tile_index_kernel wrote (its entries count the stream's rows before the window
  // too), clamped so a malformed map never addresses outside the rows
  const bool search = n <= kTileSearchRows;
  int32_t jbeg, jend;
  if (search) {
    const int32_t key = pos0 + tile * kGroup;
    jend = uniform(wave_lower_bound(rows, n, key + kGroup, lane));
    const int32_t b0 = max(0, jend - kGroup);             // positions are distinct
    const bool below = b0 + lane < jend && rows[b0 + lane] < key;
    jbeg = uniform(b0 + int32_t(__builtin_popcountll(__ballot(below))));
  } else {
    jbeg = min(max(uniform(a.tile_start[tile]) - a.row0, 0), n);
    jend = min(max(uniform(a.tile_start[tile + 1]) - a.row0, jbeg), min(n, jbeg + kGroup));
  }

  // per row: the residual (or value) as 8 packed BF16 and its position.  The predecessor row
  // is read again for the final add (an L2 hit) instead of being held in registers: the
  // register budget decides how many of these latency-bound waves a SIMD keeps in flight.
  constexpr int kR = kGroup / 8;                           // rows per lane at most
  uint4 dv[kR];
  int32_t pos[kR];
  bool bad_row = false;
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const int32_t j = jbeg + rs + 8 * i;
    pos[i] = -1;
    dv[i] = make_uint4(0, 0, 0, 0);
    if (cact && j < jend) {
      const int32_t p = rows[j] - pos0;
      if (uint32_t(p) >= uint32_t(T)) bad_row = true;      // malformed map: never address outside recon
      else pos[i] = p;
    }
  }
  uint4 rv[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    rv[i] = make_uint4(0, 0, 0, 0);
    if (pos[i] >= 0) {
      dv[i] = ld_stream(a.x + int64_t(jbeg + rs + 8 * i) * W + ch);
      if (RESID) rv[i] = *reinterpret_cast<const uint4*>(recon + int64_t(pos[i]) * W + ch);
    }
  }
  if (bad_row && a.status) atomicOr(a.status, kDevRows);
  if (search && strip == 0 && cc == 0) {
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int32_t j = jbeg + rs + 8 * i;
      if (j < jend) write_tile_index(rows, n, T, j, a.tile_start, pos0, a.row0);
    }
  }
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { mn[e] = __builtin_inff(); mx[e] = -__builtin_inff(); }
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    if (pos[i] < 0) continue;
    float v[8];
    unpack8(dv[i], v);
    if (RESID) {
      float r[8];
      unpack8(rv[i], r);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = round_bf16(v[e] - r[e]);
      dv[i] = pack8(v);                                     // exact: the values are BF16
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) { mn[e] = tmin(mn[e], v[e]); mx[e] = tmax(mx[e], v[e]); }
  }
  // Reduce-scatter over the 8 row-slot lanes of each octet (lane bits 5, 4, 3): every step
  // halves the channels a lane carries, so lane (rs, cc) ends with the extremes of channel
  // rs of its octet; it derives that channel's params alone and the octet shares them.
  const bool b2 = (rs & 4) != 0, b1 = (rs & 2) != 0, b0 = (rs & 1) != 0;
  float mn4[4], mx4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {                            // keep channels 4*b2 + q
    const float smn = b2 ? mn[q] : mn[q + 4], smx = b2 ? mx[q] : mx[q + 4];
    const float kmn = b2 ? mn[q + 4] : mn[q], kmx = b2 ? mx[q + 4] : mx[q];
    mn4[q] = tmin(kmn, __shfl_xor(smn, 32));
    mx4[q] = tmax(kmx, __shfl_xor(smx, 32));
  }
  float mn2[2], mx2[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {                            // keep channels 4*b2 + 2*b1 + q
    const float smn = b1 ? mn4[q] : mn4[q + 2], smx = b1 ? mx4[q] : mx4[q + 2];
    const float kmn = b1 ? mn4[q + 2] : mn4[q], kmx = b1 ? mx4[q + 2] : mx4[q];
    mn2[q] = tmin(kmn, __shfl_xor(smn, 16));
    mx2[q] = tmax(kmx, __shfl_xor(smx, 16));
  }
  // keep channel 4*b2 + 2*b1 + b0 = rs
  const float smn = b0 ? mn2[0] : mn2[1], smx = b0 ? mx2[0] : mx2[1];
  const float gmn = tmin(b0 ? mn2[1] : mn2[0], dpp_ror8(smn));
  const float gmx = tmax(b0 ? mx2[1] : mx2[0], dpp_ror8(smx));
  const bool empty = jend <= jbeg;
  const GroupParams own = make_params(gmn, gmx);
  const uint32_t mine = empty ? 0u : own.packed;
  if (cact) {
    st_stream32(a.params + int64_t(tile) * W + ch + rs, mine);
    if (!empty && own.err && a.status) atomicOr(a.status, own.err);
  }
  // the octet's 8 params (lane e*8 + cc holds channel e)
  float gm[8], gs[8];
  GroupParams g[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = uint32_t(__shfl(int(mine), e * 8 + cc));
    gm[e] = f16_bits_to_f32(w & 0xFFFFu);
    gs[e] = f16_bits_to_f32(w >> 16);
    g[e].m = gm[e];
    g[e].s = gs[e];
    g[e].rs = gs[e] == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(gs[e]);
  }
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    if (pos[i] < 0) continue;
    const int32_t j = jbeg + rs + 8 * i;
    uint16_t* rp = recon + int64_t(pos[i]) * W + ch;
    float v[8], k[8], out[8];
    unpack8(dv[i], v);
    codes_of_each<8>(v, g, k);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = decode(k[e], gm[e], gs[e]);
    if (RESID) {
      float r[8];
      unpack8(*reinterpret_cast<const uint4*>(rp), r);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = r[e] + round_bf16(out[e]);
    }
    st_stream32(a.codes + ((int64_t(j) * W + ch) >> 1), pack_codes8_u8(k));
    *reinterpret_cast<uint4*>(rp) = pack8(out);
  }
}

// The tile index of a compact loop (one thread per compact row), written before the
// tile-grouped K encoder runs, which reads each tile's row range from it.
__device__ __forceinline__ void tile_index_body(const EncArgs& a, uint32_t blk) {
  const int64_t j = int64_t(blk) * kThreads + threadIdx.x;
  if (j < a.n) write_tile_index(a.rows, a.n, a.T, int32_t(j), a.tile_start, a.pos0, a.row0);
}
__global__ __launch_bounds__(kThreads) void tile_index_kernel(EncArgs a) { tile_index_body(a, blockIdx.x); }

// Tile-grouped compact K loops: 4 waves per block, each on its own (tile, strip) item.
template <bool RESID>
__global__ __launch_bounds__(kThreads) void encode_k_tile_kernel(EncArgs a) {
  const uint32_t blk = xcd_remap(blockIdx.x, gridDim.x);
  encode_k_tile_body<RESID>(a, blk * (kThreads / 64) + (threadIdx.x >> 6));
}

// ---------------------------------------------------------------------------------------
// K: groups run down 64 compact rows of one (head, channel).  A block owns one 64-row band
// of a 128-channel (64 for compact loops) strip of the flattened H*D channel axis.  With
// tile groups (page-local, a.ktile) compact loops run encode_k_tile_body instead.
// Thread (rs, cc): 8 channels (16 bytes) of chunk cc, rows rs, rs + slots, ... (4 rows each
// at 128 channels, 2 at 64); the lanes of one row slot cover the strip of one row, so every
// load and store instruction covers whole rows of the strip.  Extremes: in registers over the
// thread's rows, then through LDS, where one thread per channel reduces the row slots' partial
// extremes and derives the channel's params, which every thread reads back.
// A band whose 64 rows and strip channels are all present (every band but a ragged last one,
// every strip when H*D is a multiple of the strip width) and, for a compact loop, whose rows
// all lie in [0, T) runs without per-row predicates -- buffer accesses with scalar row offsets
// and no selects; other bands take the predicated form.
// ---------------------------------------------------------------------------------------
template <bool SPARSE>
struct KShape {
  static constexpr int kCW = k_block_channels<SPARSE>();  // channels per block
  static constexpr int kChunks = kCW / 8;                 // 16-byte chunks per block row
  static constexpr int kSlots = kThreads / kChunks;       // row slots per block
  static constexpr int kRows = kGroup / kSlots;           // rows per thread
};

template <bool SPARSE>
struct KShared {
  float red[2][KShape<SPARSE>::kSlots][KShape<SPARSE>::kCW];   // partial minima, maxima
  float par[3][KShape<SPARSE>::kCW];                            // m, s, ~1/s per channel
};

// pos[i]: the X_hat row of the thread's i-th row (compact loops; -1 = not present).
template <bool RESID, bool SPARSE, bool FULL>
__device__ __forceinline__ void encode_k_band(const EncArgs& a, uint32_t strip, int32_t band,
                                              const int32_t (&pos)[KShape<SPARSE>::kRows],
                                              KShared<SPARSE>& sh) {
  using S = KShape<SPARSE>;
  const int tid = threadIdx.x;
  const int cc = tid % S::kChunks;
  const int rs = tid / S::kChunks;
  const int32_t n = a.n, T = a.T, W = a.W;
  const int32_t chunk = int32_t(strip) * S::kChunks + cc;
  const bool cact = FULL || chunk < (W >> 3);
  const uint32_t ch = uint32_t(chunk) * 8u;
  const int32_t jbeg = band * kGroup, jend = min(n, jbeg + kGroup);
  const uint32_t rowb = uint32_t(W) * 2u, crow = uint32_t(W) >> 1;
  const BufRsrc xrs = make_buf(a.x, uint32_t(n) * rowb);
  const BufRsrc rrs = make_buf(a.recon, uint32_t(T) * rowb);
  const BufRsrc crs = make_buf(a.codes, uint32_t(n) * crow);
  // row j = jbeg + rs + kSlots*i: a lane part (rs, chunk) and a scalar part (jbeg + kSlots*i)
  const uint32_t xl = uint32_t(rs) * rowb + ch * 2u;
  const uint32_t cl = uint32_t(rs) * crow + ch / 2u;
  auto xsoff = [&](int i) { return uint32_t(jbeg + S::kSlots * i) * rowb; };
  auto rl = [&](int i) { return SPARSE ? uint32_t(max(pos[i], 0)) * rowb + ch * 2u : xl; };
  auto rsoff = [&](int i) { return SPARSE ? 0u : xsoff(i); };

  bool ract[S::kRows];
#pragma unroll
  for (int i = 0; i < S::kRows; ++i)
    ract[i] = FULL || (cact && jbeg + rs + S::kSlots * i < jend && (!SPARSE || pos[i] >= 0));

  uint4 xw[S::kRows], rw[S::kRows];
#pragma unroll
  for (int i = 0; i < S::kRows; ++i) {
    if (FULL) {
      xw[i] = buf_ld128<kCacheStream>(xrs, xl, xsoff(i));
      if (RESID) rw[i] = buf_ld128(rrs, rl(i), rsoff(i));
    } else {
      xw[i] = rw[i] = make_uint4(0, 0, 0, 0);
      if (ract[i]) {
        xw[i] = buf_ld128<kCacheStream>(xrs, xl, xsoff(i));
        if (RESID) rw[i] = buf_ld128(rrs, rl(i), rsoff(i));
      }
    }
  }
  float v[S::kRows][8], r[S::kRows][8];
#pragma unroll
  for (int i = 0; i < S::kRows; ++i) {
    unpack8(xw[i], v[i]);
    if (RESID) {
      unpack8(rw[i], r[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = round_bf16(v[i][e] - r[i][e]);
    }
  }

  // the thread's extremes per channel, then one thread per channel over the row slots
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = ract[0] ? v[0][e] : __builtin_inff();
    mx[e] = ract[0] ? v[0][e] : -__builtin_inff();
#pragma unroll
    for (int i = 1; i < S::kRows; ++i) {
      mn[e] = tmin(mn[e], ract[i] ? v[i][e] : __builtin_inff());
      mx[e] = tmax(mx[e], ract[i] ? v[i][e] : -__builtin_inff());
    }
  }
  float4* dmn = reinterpret_cast<float4*>(&sh.red[0][rs][cc * 8]);
  float4* dmx = reinterpret_cast<float4*>(&sh.red[1][rs][cc * 8]);
  dmn[0] = make_float4(mn[0], mn[1], mn[2], mn[3]);
  dmn[1] = make_float4(mn[4], mn[5], mn[6], mn[7]);
  dmx[0] = make_float4(mx[0], mx[1], mx[2], mx[3]);
  dmx[1] = make_float4(mx[4], mx[5], mx[6], mx[7]);
  __syncthreads();
  if (tid < S::kCW) {
    float lo = sh.red[0][0][tid], hi = sh.red[1][0][tid];
#pragma unroll
    for (int s = 1; s < S::kSlots; ++s) {
      lo = tmin(lo, sh.red[0][s][tid]);
      hi = tmax(hi, sh.red[1][s][tid]);
    }
    const int32_t chan = int32_t(strip) * S::kCW + tid;
    const GroupParams p = make_params(lo, hi);
    sh.par[0][tid] = p.m;
    sh.par[1][tid] = p.s;
    sh.par[2][tid] = p.rs;
    if (FULL || chan < W) {
      st_stream32(a.params + int64_t(band) * W + chan, p.packed);
      if (p.err && a.status) atomicOr(a.status, p.err);
    }
  }
  __syncthreads();
  GroupParams gp[8];
  {
    const float4* pm = reinterpret_cast<const float4*>(&sh.par[0][cc * 8]);
    const float4* ps = reinterpret_cast<const float4*>(&sh.par[1][cc * 8]);
    const float4* pr = reinterpret_cast<const float4*>(&sh.par[2][cc * 8]);
    const float4 m0 = pm[0], m1 = pm[1], s0 = ps[0], s1 = ps[1], r0 = pr[0], r1 = pr[1];
    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const float rr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gp[e].m = mm[e];
      gp[e].s = ss[e];
      gp[e].rs = rr[e];
    }
  }
#pragma unroll
  for (int i = 0; i < S::kRows; ++i) {
    if (!FULL && !ract[i]) continue;
    float k[8], out[8];
    codes_of_each<8>(v[i], gp, k);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = decode(k[e], gp[e].m, gp[e].s);
    if (RESID) {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = r[i][e] + round_bf16(out[e]);
    }
    buf_st32<kCacheStream>(pack_codes8_u8(k), crs, cl, uint32_t(jbeg + S::kSlots * i) * crow);
    buf_st128(pack8(out), rrs, rl(i), rsoff(i));
  }
}

template <bool RESID, bool SPARSE>
__device__ __forceinline__ void encode_k_body(const EncArgs& a, uint32_t strip, uint32_t band_) {
  using S = KShape<SPARSE>;
  __shared__ __align__(16) KShared<SPARSE> sh;
  const int tid = threadIdx.x;
  const int cc = tid % S::kChunks;
  const int rs = tid / S::kChunks;
  const int32_t n = a.n, T = a.T, W = a.W;
  const int32_t band = int32_t(band_);
  const int32_t jbeg = band * kGroup, jend = min(n, jbeg + kGroup);
  const bool cact = int32_t(strip) * S::kChunks + cc < (W >> 3);
  bool full = jend - jbeg == kGroup && (int32_t(strip) + 1) * S::kCW <= W;
  int32_t pos[S::kRows];
  if (SPARSE) {
    bool bad = false;
#pragma unroll
    for (int i = 0; i < S::kRows; ++i) {
      const int32_t j = jbeg + rs + S::kSlots * i;
      pos[i] = -1;
      if (cact && j < jend) {
        const int32_t p = a.rows[j] - a.pos0;
        if (uint32_t(p) >= uint32_t(T)) bad = true;       // malformed map: never address outside recon
        else pos[i] = p;
      }
    }
    if (__syncthreads_or(bad)) {
      full = false;
      if (bad && a.status) atomicOr(a.status, kDevRows);
    }
    if (strip == 0 && cc == 0) {
#pragma unroll
      for (int i = 0; i < S::kRows; ++i) {
        const int32_t j = jbeg + rs + S::kSlots * i;
        if (j < jend) write_tile_index(a.rows, n, T, j, a.tile_start, a.pos0, a.row0);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < S::kRows; ++i) pos[i] = jbeg + rs + S::kSlots * i;
  }
  if (full) encode_k_band<RESID, SPARSE, true>(a, strip, band, pos, sh);
  else encode_k_band<RESID, SPARSE, false>(a, strip, band, pos, sh);
}

// Blocks run strip-fastest in XCD order: the neighbouring strips of a band write the two halves
// of the same 128-byte code lines, and so meet in one L2.
template <bool RESID, bool SPARSE>
__global__ __launch_bounds__(kThreads) void encode_k_kernel(EncArgs a) {
  uint32_t strip, band;
  xcd_block(strip, band);
  encode_k_body<RESID, SPARSE>(a, strip, band);
}

// ---------------------------------------------------------------------------------------
// V: groups run along 64 channels of one (row, head).  An item is one (compact row, head)
// pair, flattened as it = j*H + h; LPH lanes (a power of two >= D/8) cover its D channels,
// 8 channels per lane, so each 64-channel group is 8 consecutive lanes and its extremes
// come from three xor-shuffles.  Each thread handles U items spaced 256/LPH apart.
// ---------------------------------------------------------------------------------------
template <bool RESID, bool SPARSE, int LPH>
__global__ __launch_bounds__(kThreads) void encode_v_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ rows, int32_t n, int32_t T,
    int32_t H, int32_t D, uint16_t* __restrict__ recon, uint8_t* __restrict__ codes,
    uint32_t* __restrict__ params, int32_t* __restrict__ tile_start, uint32_t* __restrict__ status,
    int32_t pos0, int32_t row0) {
  constexpr int HS = kThreads / LPH;
  constexpr int U = 4;
  const int tid = threadIdx.x;
  const int w = tid & (LPH - 1);
  const int hs = tid / LPH;
  const int cph = D >> 3;
  const int S = (D + kGroup - 1) / kGroup;
  const bool wact = w < cph;
  const int64_t total = int64_t(n) * H;
  const int64_t base = int64_t(blockIdx.x) * (HS * U);

  float v[U][8];
  uint4 rv[U];
  int64_t roff[U];
  bool act[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t it = base + u * HS + hs;
    act[u] = wact && it < total;
    rv[u] = make_uint4(0, 0, 0, 0);
    roff[u] = 0;
    uint4 xv = make_uint4(0, 0, 0, 0);
    if (act[u]) {
      int64_t ro = it * D + w * 8;
      if (SPARSE) {
        const uint32_t j = uint32_t(it) / uint32_t(H);   // n*H < 2^31 (checked on the host)
        const int64_t h = it - int64_t(j) * H;
        const int32_t p = rows[j] - pos0;
        if (uint32_t(p) >= uint32_t(T)) {              // malformed map: never address outside recon
          act[u] = false;
          if (status) atomicOr(status, kDevRows);
        }
        if (h == 0 && w == 0) write_tile_index(rows, n, T, int32_t(j), tile_start, pos0, row0);
        ro = (int64_t(p) * H + h) * D + w * 8;
      }
      if (act[u]) {
        xv = ld_stream(x + it * D + w * 8);
        roff[u] = ro;
        if (RESID) rv[u] = *reinterpret_cast<const uint4*>(recon + ro);
      }
    }
    unpack8(xv, v[u]);
  }
  if (RESID) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float r[8];
      unpack8(rv[u], r);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[u][e] = round_bf16(v[u][e] - r[e]);
    }
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
    if (act[u]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) { mn = tmin(mn, v[u][e]); mx = tmax(mx, v[u][e]); }
    }
    mn = tmin(mn, __shfl_xor(mn, 1));
    mx = tmax(mx, __shfl_xor(mx, 1));
    mn = tmin(mn, __shfl_xor(mn, 2));
    mx = tmax(mx, __shfl_xor(mx, 2));
    mn = tmin(mn, __shfl_xor(mn, 4));
    mx = tmax(mx, __shfl_xor(mx, 4));
    if (!act[u]) continue;
    const int64_t it = base + u * HS + hs;
    GroupParams p = make_params(mn, mx);
    if ((w & 7) == 0) {
      st_stream32(params + it * S + (w >> 3), p.packed);
      if (p.err && status) atomicOr(status, p.err);
    }
    float k[8], out[8];
    codes_of<8>(v[u], p, k);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = decode(k[e], p.m, p.s);
    if (RESID) {
      float r[8];
      unpack8(rv[u], r);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = r[e] + round_bf16(out[e]);
    }
    st_stream32(codes + ((it * D + w * 8) >> 1), pack_codes8_u8(k));
    *reinterpret_cast<uint4*>(recon + roff[u]) = pack8(out);
  }
}

// ---------------------------------------------------------------------------------------
// V, wide rows (D % 64 == 0, H*D % 1024 == 0): a strip is 1024 channels, two halves of 64
// lanes x 8 channels, so a 64-channel group is 8 consecutive lanes and its extremes take two
// DPP quad exchanges and a half-row mirror.  Each wave walks its own run of compact rows one
// row at a time; the row index,
// rows[j] and every row offset are scalars, every access is a buffer access, and the next
// row's loads are issued before the current row is processed.
// ---------------------------------------------------------------------------------------
template <bool RESID, bool SPARSE>
__device__ __forceinline__ void encode_v_wide_body(const EncArgs& a, int32_t rows_per_wave, uint32_t bx,
                                                   uint32_t by) {
  const uint16_t* __restrict__ x = a.x;
  const int32_t* __restrict__ rows = a.rows;
  uint16_t* __restrict__ recon = a.recon;
  uint8_t* __restrict__ codes = a.codes;
  uint32_t* __restrict__ params = a.params;
  int32_t* __restrict__ tile_start = a.tile_start;
  uint32_t* __restrict__ status = a.status;
  const int32_t n = a.n, T = a.T, W = a.W;
  constexpr int kCh = 16;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int32_t j0 = (int32_t(bx) * (kThreads / 64) + wave) * rows_per_wave;
  if (j0 >= n) return;
  const int32_t j1 = min(j0 + rows_per_wave, n);
  // lane l owns channels 8l..8l+7 of each 512-channel half of the strip, so every load and
  // store instruction covers one contiguous kilobyte (a lane owning 16 adjacent channels
  // would split every cache line between two instructions, measurably slower)
  const uint32_t ch = by * 1024u + uint32_t(lane) * 8u;
  constexpr uint32_t hoff = 512u;                          // channels between the two halves
  const uint32_t xrow = uint32_t(W) * 2u, crow = uint32_t(W) / 2u, prow = uint32_t(W) / 16u;
  const BufRsrc xrs = make_buf(x, uint32_t(n) * xrow);
  const BufRsrc rrs = make_buf(recon, uint32_t(T) * xrow);
  const BufRsrc crs = make_buf(codes, uint32_t(n) * crow);
  const BufRsrc prs = make_buf(params, uint32_t(n) * prow);
  const uint32_t xv = ch * 2u, cv = ch / 2u, pv = (ch / 64u) * 4u;

  // Two register sets, used alternately; the loop is unrolled by two so every set index is
  // a compile-time constant (a runtime index would put the sets in scratch memory).
  uint4 xa[2], xb[2], ra[2], rb[2];
  int32_t pos[2];
  auto issue = [&](int32_t j, auto B) {
    constexpr int b = decltype(B)::value;
    xa[b] = buf_ld128<kCacheStream>(xrs, xv, uint32_t(j) * xrow);   // independent of the position
    xb[b] = buf_ld128<kCacheStream>(xrs, xv + 2u * hoff, uint32_t(j) * xrow);
    int32_t p = SPARSE ? uniform(rows[j]) - a.pos0 : j;
    if (SPARSE && uint32_t(p) >= uint32_t(T)) p = -1;       // malformed map: skip the row
    pos[b] = p;
    const uint32_t pr = uint32_t(max(p, 0));
    if (RESID) {
      ra[b] = buf_ld128(rrs, xv, pr * xrow);
      rb[b] = buf_ld128(rrs, xv + 2u * hoff, pr * xrow);
    }
  };
  uint32_t err = 0;
  auto process = [&](int32_t j, auto B) {
    constexpr int b = decltype(B)::value;
    const int32_t p = pos[b];
    if (SPARSE && p < 0) { err |= kDevRows; return; }
    float v[kCh], r[kCh];
    unpack8(xa[b], v);
    unpack8(xb[b], v + 8);
    if (RESID) {
      unpack8(ra[b], r);
      unpack8(rb[b], r + 8);
#pragma unroll
      for (int e = 0; e < kCh; ++e) v[e] = round_bf16(v[e] - r[e]);
    }
    // two groups per lane (one per half), each spread over 8 consecutive lanes
    float k[kCh], o[kCh];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float* vh = v + 8 * hh;
      float mn = vh[0], mx = vh[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) { mn = tmin(mn, vh[e]); mx = tmax(mx, vh[e]); }
      mn = tmin(mn, dpp_xor1(mn));
      mx = tmax(mx, dpp_xor1(mx));
      mn = tmin(mn, dpp_xor2(mn));
      mx = tmax(mx, dpp_xor2(mx));
      mn = tmin(mn, dpp_half_mirror(mn));
      mx = tmax(mx, dpp_half_mirror(mx));
      const GroupParams gp = make_params(mn, mx);
      err |= gp.err;
      codes_of<8>(vh, gp, k + 8 * hh);
      if ((lane & 7) == 0) buf_st32<kCacheStream>(gp.packed, prs, pv + hh * (hoff / 64u) * 4u, uint32_t(j) * prow);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[8 * hh + e] = decode(k[8 * hh + e], gp.m, gp.s);
        if (RESID) o[8 * hh + e] = r[8 * hh + e] + round_bf16(o[8 * hh + e]);
      }
    }
    buf_st32<kCacheStream>(pack_codes8_u8(k), crs, cv, uint32_t(j) * crow);
    buf_st32<kCacheStream>(pack_codes8_u8(k + 8), crs, cv + hoff / 2u, uint32_t(j) * crow);
    buf_st128(pack8(o), rrs, xv, uint32_t(p) * xrow);
    buf_st128(pack8(o + 8), rrs, xv + 2u * hoff, uint32_t(p) * xrow);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  issue(j0, B0{});
  if (!SPARSE) {
    for (int32_t j = j0; j < j1; j += 2) {
      if (j + 1 < j1) issue(j + 1, B1{});
      process(j, B0{});
      if (j + 1 >= j1) break;
      if (j + 2 < j1) issue(j + 2, B0{});
      process(j + 1, B1{});
    }
  } else {
    // Compact loops: inside the loop every row is processed with exactly one younger set of
    // loads in flight, and the last one or two rows take their own code path (a row reached
    // both with and without a younger set makes the wait before it a wait for every
    // outstanding load, the prefetch included).
    int32_t j = j0;
    for (; j + 2 < j1; j += 2) {
      issue(j + 1, B1{});
      process(j, B0{});
      issue(j + 2, B0{});
      process(j + 1, B1{});
    }
    if (j + 1 < j1) {
      issue(j + 1, B1{});
      process(j, B0{});
      process(j + 1, B1{});
    } else {
      process(j, B0{});
    }
    // The tile index entries of the wave's rows, once its rows are done: stores of a varying
    // count inside the row loop would likewise turn the waits there into waits for every
    // outstanding load.
    if (by == 0) {
      for (int32_t jb = j0; jb < j1; jb += 64)
        if (jb + lane < j1) write_tile_index(rows, n, T, jb + lane, tile_start, a.pos0, a.row0);
    }
  }
  if (err && status) atomicOr(status, err);
}

template <bool RESID, bool SPARSE>
__global__ __launch_bounds__(kThreads) void encode_v_wide_kernel(EncArgs a, int32_t rows_per_wave) {
  encode_v_wide_body<RESID, SPARSE>(a, rows_per_wave, blockIdx.x, blockIdx.y);
}

static bool v_wide_ok(int32_t H, int32_t D) { return D % 64 == 0 && (H * D) % 1024 == 0; }

// Rows per wave of the wide V encoder: about kVWideWaves waves per launch -- many short waves
// (one or two rows each) keep the most loads in flight and let the wave scheduler hide their
// latency.
// (host and device: the batched kernel derives each unit's grid from its sizes)
__host__ __device__ inline int32_t v_wide_rpw(int32_t n, int32_t W) {
  const int64_t per_wave = (int64_t(n) * (W / 1024) + kVWideWaves - 1) / kVWideWaves;
  return int32_t(per_wave < 1 ? 1 : per_wave);
}
__host__ __device__ inline uint32_t v_wide_grid_x(int32_t n, int32_t rpw) {
  const int32_t waves = (n + rpw - 1) / rpw;
  return uint32_t((waves + 3) / 4);
}
static dim3 v_wide_grid(int32_t n, int32_t W, int32_t rpw) { return dim3(v_wide_grid_x(n, rpw), unsigned(W / 1024)); }
// x: channel strips, y: 64-row bands; tile groups of a compact loop: one wave per (tile,
// 64-channel strip), 4 waves per block along x
__host__ __device__ inline uint32_t k_grid_x(int32_t W, int32_t T, bool sparse, bool ktile) {
  if (sparse && ktile) {
    const int64_t waves = int64_t((W / 8 + 7) / 8) * ((T + kGroup - 1) / kGroup);
    return uint32_t((waves + 3) / 4);
  }
  const int chunks = (sparse ? k_block_channels<true>() : k_block_channels<false>()) / 8;
  return uint32_t((W / 8 + chunks - 1) / chunks);
}
static dim3 k_grid(const EncArgs& a, bool sparse) {
  if (sparse && a.ktile) return dim3(k_grid_x(a.W, a.T, true, true), 1);
  return dim3(k_grid_x(a.W, a.T, sparse, false), unsigned((a.n + kGroup - 1) / kGroup));
}

template <bool RESID, bool SPARSE>
static hipError_t launch_v_wide(const EncArgs& a, hipStream_t stream) {
  const int32_t rpw = v_wide_rpw(a.n, a.W);
  hipLaunchKernelGGL((encode_v_wide_kernel<RESID, SPARSE>), v_wide_grid(a.n, a.W, rpw), dim3(kThreads), 0,
                     stream, a, rpw);
  return hipGetLastError();
}

template <bool RESID, bool SPARSE>
static hipError_t launch_v(const EncArgs& a, int32_t H, int32_t D, hipStream_t stream) {
  const int cph = D / 8;
  const int lph = cph <= 8 ? 8 : cph <= 16 ? 16 : cph <= 32 ? 32 : 64;
  const int per_block = (kThreads / lph) * 4;
  const int64_t items = int64_t(a.n) * H;
  const dim3 grid(unsigned((items + per_block - 1) / per_block));
#define FLK_LAUNCH_V(L)                                                                          \
  hipLaunchKernelGGL((encode_v_kernel<RESID, SPARSE, L>), grid, dim3(kThreads), 0, stream, a.x,   \
                     a.rows, a.n, a.T, H, D, a.recon, a.codes, a.params, a.tile_start, a.status, \
                     a.pos0, a.row0)
  switch (lph) {
    case 8: FLK_LAUNCH_V(8); break;
    case 16: FLK_LAUNCH_V(16); break;
    case 32: FLK_LAUNCH_V(32); break;
    default: FLK_LAUNCH_V(64); break;
  }
#undef FLK_LAUNCH_V
  return hipGetLastError();
}

template <bool RESID, bool SPARSE>
static hipError_t launch_k(const EncArgs& a, hipStream_t stream) {
  if (SPARSE && a.ktile) {
    if (a.n > kTileSearchRows)
      hipLaunchKernelGGL(tile_index_kernel, dim3(unsigned((a.n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                         stream, a);
    hipLaunchKernelGGL((encode_k_tile_kernel<RESID>), k_grid(a, SPARSE), dim3(kThreads), 0, stream, a);
  } else
    hipLaunchKernelGGL((encode_k_kernel<RESID, SPARSE>), k_grid(a, SPARSE), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_encode(int kind, bool resid, const EncArgs& a, int32_t H, int32_t D, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const bool sparse = a.rows != nullptr;
  if (kind == FLK_KIND_K) {
    if (!resid) return launch_k<false, false>(a, stream);
    if (!sparse) return launch_k<true, false>(a, stream);
    return launch_k<true, true>(a, stream);
  }
  if (v_wide_ok(H, D)) {
    if (!resid) return launch_v_wide<false, false>(a, stream);
    if (!sparse) return launch_v_wide<true, false>(a, stream);
    return launch_v_wide<true, true>(a, stream);
  }
  if (!resid) return launch_v<false, false>(a, H, D, stream);
  if (!sparse) return launch_v<true, false>(a, H, D, stream);
  return launch_v<true, true>(a, H, D, stream);
}

__global__ __launch_bounds__(kThreads) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t count, uint32_t value) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i < count) p[i] = value;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  if (p == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(unsigned((count + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     p, count, value);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Batched encode: one launch runs the same loop type (base, dense residual or compact
// residual) for up to kEncBatch tensors, K and V mixed.  Blocks are numbered unit after unit;
// a block finds its unit with a scan of the (scalar) block offsets and runs that kind's body.
// V tensors take the wide body only, so a V unit needs D % 64 == 0 and H*D % 1024 == 0.
// ---------------------------------------------------------------------------------------
// What a unit's encode needs beyond the batch's shared fields (status word, K grouping),
// packed so that kEncBatch units fit the kernel-argument space; its kind is a bit of the
// batch and its grid is derived from its sizes, as the host derived it.
struct EncUnit {
  const uint16_t* x;
  const int32_t* rows;
  uint16_t* recon;
  uint8_t* codes;
  uint32_t* params;
  int32_t* tile_start;
  int32_t n, T, W, pos0, row0;
  uint32_t block0;    // first block of the unit in the launch
};
struct EncBatch {
  uint32_t* status;
  uint64_t v_units;   // bit i: unit i is a V tensor
  int32_t n_units;
  int32_t ktile;      // the K units' grouping (one K descriptor per call)
  EncUnit u[kEncBatch];
};

static_assert(kEncBatch <= 64, "one kind bit per unit");
static_assert(sizeof(EncBatch) <= 4096, "a batch travels as kernel arguments (4 KiB at most)");

__device__ __forceinline__ EncArgs unit_args(const EncBatch& b, const EncUnit& u, bool is_v) {
  return EncArgs{u.x, u.rows, u.recon, u.codes, u.params, u.tile_start, b.status, u.n, u.T, u.W, u.pos0, u.row0,
                 is_v ? 0 : b.ktile};
}

// The unit of a block: the last unit whose first block is at or below it (a scan of scalars).
__device__ __forceinline__ int batch_unit(const EncBatch& b, uint32_t bid) {
  int ui = 0;
#pragma unroll
  for (int i = 1; i < kEncBatch; ++i)
    if (i < b.n_units && bid >= b.u[i].block0) ui = i;
  return ui;
}

template <bool RESID, bool SPARSE, bool KTILE>
__global__ __launch_bounds__(kThreads) void encode_batch_kernel(EncBatch b) {
  const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int ui = batch_unit(b, bid);
  const EncUnit& u = b.u[ui];
  const bool is_v = ((b.v_units >> ui) & 1u) != 0;
  const EncArgs a = unit_args(b, u, is_v);
  const int32_t rpw = is_v ? v_wide_rpw(u.n, u.W) : 0;
  const uint32_t gx = is_v ? v_wide_grid_x(u.n, rpw) : k_grid_x(u.W, u.T, SPARSE, KTILE);
  const uint32_t lb = bid - u.block0;
  const uint32_t by = lb / gx, bx = lb - by * gx;
  if (!is_v) {
    if (SPARSE && KTILE) encode_k_tile_body<RESID>(a, bx * (kThreads / 64) + (threadIdx.x >> 6));
    else encode_k_body<RESID, SPARSE>(a, bx, by);
  } else {
    encode_v_wide_body<RESID, SPARSE>(a, rpw, bx, by);
  }
}

// The tile indexes of a batch's tile-grouped compact K units, before their encode.
__global__ __launch_bounds__(kThreads) void tile_index_batch_kernel(EncBatch b) {
  const int ui = batch_unit(b, blockIdx.x);
  tile_index_body(unit_args(b, b.u[ui], false), blockIdx.x - b.u[ui].block0);
}

bool encode_batchable(int kind, int32_t H, int32_t D) { return kind == FLK_KIND_K || v_wide_ok(H, D); }

hipError_t launch_encode_batch(bool resid, bool sparse, const EncArgs* args, const int* kinds, int n_units,
                               hipStream_t stream) {
  for (int u0 = 0; u0 < n_units; u0 += kEncBatch) {
    EncBatch b{};
    uint32_t blocks = 0;
    bool ktile = false;                         // the K units' grouping (one K descriptor per call)
    for (int i = u0; i < n_units && i < u0 + kEncBatch; ++i) {
      const EncArgs& a = args[i];
      if (a.n <= 0) continue;
      if (kinds[i] == FLK_KIND_K && a.ktile) ktile = true;
      if (a.status) b.status = a.status;        // one status word per call
      const int k = b.n_units++;
      b.u[k] = EncUnit{a.x, a.rows, a.recon, a.codes, a.params, a.tile_start, a.n, a.T, a.W, a.pos0, a.row0, blocks};
      dim3 g;
      if (kinds[i] == FLK_KIND_K) {
        g = k_grid(a, sparse);
      } else {
        b.v_units |= uint64_t(1) << k;
        g = v_wide_grid(a.n, a.W, v_wide_rpw(a.n, a.W));
      }
      blocks += g.x * g.y;
    }
    b.ktile = ktile ? 1 : 0;
    if (blocks == 0) continue;
    if (sparse && ktile) {
      EncBatch tb{};
      tb.status = b.status;
      tb.ktile = 1;
      uint32_t tblocks = 0;
      for (int i = 0; i < b.n_units; ++i) {
        if (((b.v_units >> i) & 1u) != 0 || b.u[i].n <= kTileSearchRows) continue;
        EncUnit& e = tb.u[tb.n_units++];
        e = b.u[i];
        e.block0 = tblocks;
        tblocks += uint32_t((e.n + kThreads - 1) / kThreads);
      }
      if (tblocks > 0)
        hipLaunchKernelGGL(tile_index_batch_kernel, dim3(tblocks), dim3(kThreads), 0, stream, tb);
    }
    if (!resid)
      hipLaunchKernelGGL((encode_batch_kernel<false, false, false>), dim3(blocks), dim3(kThreads), 0, stream, b);
    else if (!sparse)
      hipLaunchKernelGGL((encode_batch_kernel<true, false, false>), dim3(blocks), dim3(kThreads), 0, stream, b);
    else if (!ktile)
      hipLaunchKernelGGL((encode_batch_kernel<true, true, false>), dim3(blocks), dim3(kThreads), 0, stream, b);
    else
      hipLaunchKernelGGL((encode_batch_kernel<true, true, true>), dim3(blocks), dim3(kThreads), 0, stream, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace flk
