// flk_attn_split.hip -- decode attention over INT4 packed chains in two passes over the tokens
// (FlashLoop RFC, vllm-rlt #156, section 3.3: readers consume the packed base/residual tiles
// directly during QK and PV).
//
// Pass 1 (attn_scores_kernel) decodes K_hat bit for bit as the encoder left it -- the BF16
// rounding after every loop of the chain matters here: a sharp softmax turns a one-ulp change
// of a key into a visible change of the output -- and writes every scaled score
// s[head][position] and, per block, each query head's maximum score.
// Pass 2 (attn_pv_kernel) takes V straight from the codes.  A V loop's contribution is linear
// in its codes, V_hat_l = min + scale * code per (row, 64-channel group), so
// sum_t p_t V_l[t] = sum_t p_t min_t + sum_t (p_t scale_t) code_t: the codes go to the MFMA
// as binary16 1024 + code (a nibble ORed into 0x6400), the B operand is p * scale in
// binary16, and the minima and the 1024 offset are a per-(head, group) correction accumulated
// with dot2.  The loops are walked one at a time over their own compact rows, so no row the
// loop does not list is ever touched.  Leaving out the chain's intermediate BF16 roundings of
// V_hat changes the output by a few 1e-3 relative (errors average over the tokens), against
// 1e-1 for K.
// Both passes use the same blocks (split, KV head), so the block maximum of pass 1 is the
// reference of pass 2's probabilities and pass 2's partial (max, sum, O) per block merges in
// the same combine kernel as the fused path.  A BF16 tail (a rolling cache's recent tokens)
// is read as stored, 16 tokens per wave, in both passes; its scores follow the packed ones.
#include "flk_attn_common.h"

namespace flk {

// ---- pass 1: scores ------------------------------------------------------------------------
//
// A 4-bit code read as a binary16 bit pattern is the denormal code * 2^-24, so v_fma_mix_f32
// takes it straight from a 16-bit half of the code word, with no conversion instruction.  The
// scale is staged as the binary32 s * 2^24 (exact: a power-of-two multiple of a binary16
// value) and the minimum as its binary16 bits; the product is then exactly code * s, and the
// fma gives RN(code * s + m), the value the encoder's decode gives.
// A lane's four items are four consecutive octets, 4*kb .. 4*kb+3 (32 channels, one 16-byte
// code load per loop); the query operand takes the same channels, so the MFMA sums the same
// products.

#ifndef FLK_SCORES_OCC
#define FLK_SCORES_OCC 4   // waves per SIMD the scores pass's register budget must allow
#endif

constexpr int kKsRow = 36;                 // 32 scales + 4 pad: block b starts at bank 4b
constexpr int kKmRow = 40;                 // 32 minima + 8 pad: blocks start at banks 0, 20, 8, 28

template <int NL>
struct ScoreLds {
  // Per loop and rowgroup parity, the 128 channels in 4 blocks of 32 (a lane block's channels),
  // each block padded so the 4 lane blocks' reads of one instruction hit different banks:
  float ks[NL][2][4][kKsRow];              // K scale * 2^24 (binary32)
  uint16_t km[NL][2][4][kKmRow];           // K minimum, FP16 bits
  int32_t map[NL][kGroup];                 // [loop][position in tile] -> compact row, -1 absent
  int32_t perm[kGroup];                    // tile positions grouped by which loops list them
};

// One slice's loads: per loop the lane's compact row (-1: the loop does not list the token)
// and its 16 code bytes (octets 4*kb .. 4*kb+3).  Dense loops read position min(t, T - 1): a
// lane past the end decodes a copy of the last row, whose score goes nowhere (an MFMA output
// row depends on its own input row only).  A compact loop's absent token reads row 0 and
// skips the decode.  So every load is unconditional and no register needs a default value.
// An FP4 loop (FMT) adds the lane's block scale bytes: NVFP4 the E4M3 bytes of its two 16-channel
// blocks (2 kb, 2 kb + 1), MXFP4 the E8M0 byte of its 32-channel block kb.
template <int NL>
struct KSliceLoads {
  int32_t j[NL];
  uint4 cw[NL];
  uint32_t sw[NL];
};

template <int NL, int FMT>
__device__ __forceinline__ void issue_k_slice(const ChainArgs& c, const TileRows<NL>& r, int32_t t, int32_t T,
                                              int32_t H, int32_t h, int kb, const int32_t (*map)[kGroup],
                                              int tk, KSliceLoads<NL>& ld) {
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    ld.j[l] = r.dense[l] ? min(t, T - 1) : map[l][tk];
    const uint32_t item = uint32_t(max(ld.j[l], 0)) * uint32_t(H) + uint32_t(h);
    ld.cw[l] = *reinterpret_cast<const uint4*>(c.s[l].codes + (item * (kAttnD / 2) + 16u * uint32_t(kb)));
    if (loop_fp4<FMT>(l)) {
      const uint8_t* pb = reinterpret_cast<const uint8_t*>(c.s[l].params);
      ld.sw[l] = loop_mx<FMT>(l)
                     ? uint32_t(pb[item * 4u + uint32_t(kb)])
                     : uint32_t(*reinterpret_cast<const uint16_t*>(pb + 16u + item * 8u + 2u * uint32_t(kb)));
    }
  }
}

// K_hat of the lane's item i (8 channels), packed BF16 for the MFMA: the chain's
// bf16(... bf16(bf16(base) + bf16(d2)) ... + bf16(dR)) with d = RN(code * s + m) for an INT4
// loop and d = RN(e2m1 * block scale) for an FP4 loop (as flk_reconstruct decodes them).
template <int NL, int FMT>
__device__ __forceinline__ uint4 decode_k_item(const ChainArgs& c, const KSliceLoads<NL>& ld, int kb, int i,
                                               const ScoreLds<NL>& L, uint32_t ones, const float* gsc) {
  float acc[8];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (l > 0 && ld.j[l] < 0) continue;                  // the base is dense: every lane decodes it
    const uint32_t cwi = i == 0 ? ld.cw[l].x : i == 1 ? ld.cw[l].y : i == 2 ? ld.cw[l].z : ld.cw[l].w;
    if (loop_fp4<FMT>(l)) {
      float d[8], bs;
      if (loop_mx<FMT>(l)) {
        bs = fp4_e8m0_value(ld.sw[l] & 0xFFu);
      } else {                                           // item i lies in the lane's block i / 2
        const fp4_f32x2 s2 = e4m3x2_value(ld.sw[l]);
        bs = (i < 2 ? s2.x : s2.y) * gsc[l];
      }
      fp4_decode8(cwi, bs, d);
      if (l == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = d[e];
      } else {
        add_rounded_bf16x8(acc, d, ones);
      }
      continue;
    }
    const int rg = c.ktile ? 0 : (ld.j[l] / kGroup) & 1;   // staged by rowgroup parity
    const float4 s0 = *reinterpret_cast<const float4*>(&L.ks[l][rg][kb][8 * i]);
    const float4 s1 = *reinterpret_cast<const float4*>(&L.ks[l][rg][kb][8 * i + 4]);
    const uint4 mw = *reinterpret_cast<const uint4*>(&L.km[l][rg][kb][8 * i]);
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const uint32_t mv[4] = {mw.x, mw.y, mw.z, mw.w};
    uint32_t wq[4];
    codes8_to_f16_halves(cwi, wq);
    float d[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d[q] = __builtin_fmaf(f16lo(wq[q]), sv[q], (q & 1) ? f16hi(mv[q >> 1]) : f16lo(mv[q >> 1]));
      d[q + 4] = __builtin_fmaf(f16hi(wq[q]), sv[q + 4], (q & 1) ? f16hi(mv[2 + (q >> 1)]) : f16lo(mv[2 + (q >> 1)]));
    }
    if (l == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = d[e];
    } else {
      add_rounded_bf16x8(acc, d, ones);
    }
  }
  return round_bf16x8(acc);
}

// One slice: decode K_hat, S^T = K_hat Q^T on the MFMA, the scaled scores to their positions'
// entries of the scores rows and into the running maximum.
template <int NL, int FMT>
__device__ __forceinline__ void score_slice(const ChainArgs& kc, const KSliceLoads<NL>& ld, int kb,
                                            const ScoreLds<NL>& L, uint32_t ones, const bf16x8_t qb[4], int sl,
                                            int32_t n_valid, int32_t t0, int n, int32_t G, float scale,
                                            float* srow, float& mx, const float* gsc) {
  // each item goes to the MFMA as soon as it is decoded, so one item's registers are live
  float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 item = decode_k_item<NL, FMT>(kc, ld, kb, ks, L, ones, gsc);
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, item), qb[ks], sacc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = 16 * sl + 4 * kb + i;
    if (slot < n_valid) {
      const float sc = sacc[i] * scale;
      mx = fmaxf(mx, sc);
      if (n < G) srow[t0 + L.perm[slot]] = sc;
    }
  }
}

// TAIL: the call has a BF16 tail (an instance of its own, so the packed-only loop keeps its
// register allocation).
template <int NL, bool TAIL, int FMT>
__global__ __launch_bounds__(kAThreads, FLK_SCORES_OCC) void attn_scores_kernel(ChainArgs kc, int32_t T, int32_t H, int32_t G,
                                                                   const uint16_t* __restrict__ q, float scale,
                                                                   int32_t wph, float* __restrict__ scores,
                                                                   float* __restrict__ block_max,
                                                                   const uint16_t* __restrict__ kt, int32_t tail_len) {
  __shared__ __attribute__((aligned(16))) ScoreLds<NL> s_lds[kAWaves];
  __shared__ float s_max[kAWaves][kMaxG];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;
  const int kb = lane >> 4;
  // the block order of the fused kernel: split-major, head-minor, contiguous per XCD
  const uint32_t lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int32_t split = int32_t(lin / gridDim.y);
  const int32_t h = int32_t(lin % gridDim.y);
  const int32_t Hq = H * G;
  const int32_t ptiles = (T + kGroup - 1) / kGroup;
  const int32_t w = split * kAWaves + wave;
  const int32_t base = ptiles / wph, extra = ptiles - base * wph;
  const int32_t tile0 = w < wph ? w * base + min(w, extra) : ptiles;
  const int32_t tile1 = w < wph ? tile0 + base + (w < extra ? 1 : 0) : ptiles;
  ScoreLds<NL>& L = s_lds[wave];
  const int64_t Tpad = (int64_t(T) + (TAIL ? tail_len : 0) + 3) & ~int64_t(3);   // positions T.. hold the tail
  const uint32_t ones = bf16_ones();

  // query operand of k-step ks: channels 32*kb + 8*ks .. +7, the channels of the lane's item ks
  bf16x8_t qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 qw = make_uint4(0, 0, 0, 0);
    if (n < G) qw = *reinterpret_cast<const uint4*>(q + int64_t(h * G + n) * kAttnD + 32 * kb + 8 * ks);
    qb[ks] = __builtin_bit_cast(bf16x8_t, qw);
  }

  float* srow = scores + int64_t(h * G + (n < G ? n : 0)) * Tpad;
  float mx = -__builtin_inff();
  // the NVFP4 loops' stream scales, read once (the scores stores in the loop below would
  // otherwise make the compiler reload them for every slice)
  float gsc[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) gsc[l] = loop_nv<FMT>(l) && l < kc.n_loops ? __uint_as_float(kc.s[l].params[0]) : 1.0f;
  // The BF16 tail, read as stored, in 16-token slices: slice s goes to waves s, s + wph, ...
  // of every head (a small addition to many waves); its scores follow the packed positions.
  const int32_t tail_slices = (tail_len + 15) / 16;
  for (int32_t ts = w; TAIL && w < wph && ts < tail_slices; ts += wph) {
    const int32_t nv = min(16, tail_len - 16 * ts);
    const int64_t b = (int64_t(16 * ts + n) * H + h) * kAttnD + 32 * kb;
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 item = n < nv ? *reinterpret_cast<const uint4*>(kt + b + 8 * ks) : make_uint4(0, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, item), qb[ks], sacc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 4 * kb + i;
      if (slot < nv) {
        const float sc = sacc[i] * scale;
        mx = fmaxf(mx, sc);
        if (n < G) srow[int64_t(T) + 16 * ts + slot] = sc;
      }
    }
  }
  for (int32_t tile = tile0; tile < tile1; ++tile) {
    const int32_t t0 = tile * kGroup;
    const TileRows<NL> rk = tile_rows<NL>(kc, tile, T);
    wave_sync();                                          // the previous tile's LDS reads are done
    build_maps<NL>(kc, rk, t0, L.map, lane);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (l >= kc.n_loops || loop_fp4<FMT>(l)) continue;  // an FP4 loop's scales come per token
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        int32_t row;                                      // the parameter row staged in slot r
        if (kc.ktile) {
          if (r == 1 || rk.hi[l] <= rk.lo[l]) continue;
          row = tile;
        } else {
          const int32_t nrg = (kc.s[l].n + kGroup - 1) / kGroup;
          row = rk.lo[l] / kGroup + r;
          if ((r == 1 && rk.dense[l]) || row >= nrg) continue;
        }
        const int slot = kc.ktile ? 0 : (row & 1);
        const uint2 pw = *reinterpret_cast<const uint2*>(kc.s[l].params + (uint32_t(row) * uint32_t(H) + uint32_t(h)) * kAttnD + 2 * lane);
        // word = (min16, scale16): scale * 2^24 in binary32, the minima as they are
        *reinterpret_cast<float2*>(&L.ks[l][slot][lane >> 4][(2 * lane) & 31]) = make_float2(f16hi(pw.x) * kCodeScale,
                                                                           f16hi(pw.y) * kCodeScale);
        *reinterpret_cast<uint32_t*>(&L.km[l][slot][lane >> 4][(2 * lane) & 31]) = __builtin_amdgcn_perm(pw.y, pw.x, 0x05040100u);
      }
    }
    // positions listed by the same loops sit together, so a loop none of a slice's tokens has
    // is skipped by the whole wave; positions past T go last
    const int32_t n_valid = min(kGroup, T - t0);
    {
      uint32_t key = 0;
#pragma unroll
      for (int l = 1; l < NL; ++l)
        if (l < kc.n_loops && !rk.dense[l] && L.map[l][lane] >= 0) key |= 1u << l;
      const bool valid = lane < n_valid;
      const uint64_t below = (uint64_t(1) << lane) - 1;
      uint64_t remaining = __ballot(valid);
      int nb = 0, rank = 0;
      while (remaining) {
        const int leader = __builtin_ctzll(remaining);
        const uint32_t k = __builtin_amdgcn_readlane(key, leader);
        const uint64_t grp = __ballot(valid && key == k);
        if (valid && key == k) rank = nb + __builtin_popcountll(grp & below);
        nb += __builtin_popcountll(grp);
        remaining &= ~grp;
      }
      if (!valid) rank = lane;
      L.perm[rank] = lane;
    }
    wave_sync();
    // two slices' loads in flight: slice sl + 1 is requested before slice sl is decoded (the
    // loop takes the slices in pairs, so each slice's loads have fixed registers)
    KSliceLoads<NL> la, lb;
    issue_k_slice<NL, FMT>(kc, rk, t0 + L.perm[n], T, H, h, kb, L.map, L.perm[n], la);
#pragma nounroll
    for (int sl = 0; sl * 16 < n_valid; sl += 2) {
      const bool second = (sl + 1) * 16 < n_valid;
      if (second) {
        const int tk = L.perm[16 * (sl + 1) + n];
        issue_k_slice<NL, FMT>(kc, rk, t0 + tk, T, H, h, kb, L.map, tk, lb);
      }
      score_slice<NL, FMT>(kc, la, kb, L, ones, qb, sl, n_valid, t0, n, G, scale, srow, mx, gsc);
      if (!second) break;
      if ((sl + 2) * 16 < n_valid) {
        const int tk = L.perm[16 * (sl + 2) + n];
        issue_k_slice<NL, FMT>(kc, rk, t0 + tk, T, H, h, kb, L.map, tk, la);
      }
      score_slice<NL, FMT>(kc, lb, kb, L, ones, qb, sl + 1, n_valid, t0, n, G, scale, srow, mx, gsc);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (kb == 0) s_max[wave][n] = mx;
  __syncthreads();
  if (int(threadIdx.x) < G) {
    float m = -__builtin_inff();
#pragma unroll
    for (int wv = 0; wv < kAWaves; ++wv) m = fmaxf(m, s_max[wv][threadIdx.x]);
    block_max[int64_t(split) * Hq + h * G + int(threadIdx.x)] = m;
  }
}

// ---- pass 2: PV from the V codes -----------------------------------------------------------

// One wave's staging of a slice: 16 code rows (chunks swizzled, see pv_chunk) and 16 parameter
// rows (words 32..63 stay unused).  A wave stages kPvBatch slices at a time.
//
// Token k = 4 kb + r of the MFMA (lane block kb, its r-th token) is staged row 4 r + kb, so one
// read instruction's four rows (kb = 0..3) are consecutive: two even and two odd rows, which
// lie in the two halves of the LDS banks (64-byte rows).  The two rows of a parity differ in
// bit 1 of the row index, and pv_chunk moves their 16-byte chunks two places apart, so the 32
// dwords of an instruction's reads fall in 32 distinct banks.
__device__ __forceinline__ int pv_chunk(int row, int q) { return q ^ (((row >> 1) & 1) << 1); }
struct PvStage {
  uint8_t codes[16][kAttnD / 2];
  uint32_t params[64];
};
#ifndef FLK_PV_BATCH
#define FLK_PV_BATCH 4
#endif
constexpr int kPvBatch = FLK_PV_BATCH;
static_assert(sizeof(PvStage) * kPvBatch >= 16 * kAttnD * sizeof(uint16_t), "a wave's staging holds a BF16 tail slice");
union PvLds {
  PvStage stage[kAWaves][kPvBatch];
  struct {
    float o[kAWaves][kMaxG][kAttnD];
    float l[kAWaves][kMaxG];
  } merge;
};

template <int NL, int FMT>
__global__ __launch_bounds__(kAThreads, 4) void attn_pv_kernel(ChainArgs vc, int32_t T, int32_t H, int32_t G,
                                                               const float* __restrict__ scores,
                                                               const float* __restrict__ block_max, int32_t wph,
                                                               float* __restrict__ ws_ml, float* __restrict__ ws_o,
                                                               const uint16_t* __restrict__ vt, int32_t tail_len) {
  __shared__ __attribute__((aligned(16))) PvLds s_lds;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;
  const int kb = lane >> 4;
  const uint32_t lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int32_t split = int32_t(lin / gridDim.y);
  const int32_t h = int32_t(lin % gridDim.y);
  const int32_t Hq = H * G;
  const int32_t ptiles = (T + kGroup - 1) / kGroup;
  const int32_t w = split * kAWaves + wave;
  const int32_t base = ptiles / wph, extra = ptiles - base * wph;
  const int32_t tile0 = w < wph ? w * base + min(w, extra) : ptiles;
  const int32_t tile1 = w < wph ? tile0 + base + (w < extra ? 1 : 0) : ptiles;
  PvStage* Sw = s_lds.stage[wave];
  const int64_t Tpad = (int64_t(T) + tail_len + 3) & ~int64_t(3);
  const int32_t P0 = tile0 * kGroup, P1 = min(tile1 * kGroup, T);

  // the block's maximum score of this lane's query head (pass 1); probabilities are relative to it
  const float m = n < G ? block_max[int64_t(split) * Hq + h * G + n] : 0.0f;
  // the KV head's scores rows, one resource; this lane's row starts srow_off floats in
  const BufRsrc sb_rsrc = make_buf(scores + int64_t(h) * G * Tpad, uint32_t(int64_t(G) * Tpad * 4));
  const uint32_t srow_off = uint32_t(n < G ? n : 0) * uint32_t(Tpad);
  const bool head_live = n < G && m != -__builtin_inff();

  float4_t o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float vmin[2] = {0.0f, 0.0f};   // per V group: sum p * min - 1024 * sum (p * scale) over this lane's rows
  float lsum = 0.0f;
  const f16x2_t m1024 = __builtin_bit_cast(f16x2_t, 0xE400E400u);   // (-1024, -1024)
  const uint32_t nib = opaque(0x000F000Fu);                        // a VGPR operand: one v_and_or per word

  // this lane's staging slots: 16 bytes of code row crow (chunk cq), parameter word of prow
  const int crow = lane >> 2, prow = (lane & 31) >> 1;
  const int cq = pv_chunk(crow, lane & 3);

  // The BF16 tail, as the scores pass split it: per 16-token slice, its V rows through the
  // wave's staging area in LDS (16 rows of 128 BF16), O^T += V^T P^T on the BF16 MFMA
  const int32_t tail_slices = (tail_len + 15) / 16;
  for (int32_t ts = w; w < wph && ts < tail_slices; ts += wph) {
    const int32_t nv = min(16, tail_len - 16 * ts);
    uint16_t (*vs)[kAttnD] = reinterpret_cast<uint16_t (*)[kAttnD]>(&Sw[0]);
    wave_sync();                                          // earlier reads of the staging area are done
    {
      const int row = lane >> 2, c0 = 32 * (lane & 3);
      const int64_t b = (int64_t(16 * ts + row) * H + h) * kAttnD + c0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&vs[row][c0 + 8 * i]) =
            row < nv ? *reinterpret_cast<const uint4*>(vt + b + 8 * i) : make_uint4(0, 0, 0, 0);
    }
    short4_t pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t k = 4 * kb + r;
      const float p = k < nv && head_live ? __expf(__uint_as_float(buf_ld32(sb_rsrc, (srow_off + uint32_t(T + 16 * ts + k)) * 4u, 0u)) - m)
                                          : 0.0f;
      lsum += p;
      pb[r] = short(__builtin_bit_cast(uint16_t, (__bf16)p));
    }
    wave_sync();
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      short4_t a;
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = short(vs[4 * kb + r][pv_channel(mt, n)]);
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[mt], 0, 0, 0);
    }
  }

#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (l >= vc.n_loops || P0 >= P1) continue;
    const StreamArgs st = vc.s[l];
    const bool dense = st.rows == nullptr;
    // the loop's compact rows of positions [P0, P1)
    const int32_t a = dense ? P0 : uniform(st.tile_start[tile0]);
    const int32_t b = dense ? P1 : uniform(st.tile_start[tile1]);
    const uint32_t nbytes = uint32_t(st.n) * uint32_t(H);
    const BufRsrc cb = make_buf(st.codes, nbytes * (kAttnD / 2));
    // parameter bytes per row: INT4 two (min, scale) words; NVFP4 8 E4M3 bytes after a 16-byte
    // header; MXFP4 4 E8M0 bytes (staged in the row's first word)
    const bool fp4 = loop_fp4<FMT>(l), mx = loop_mx<FMT>(l);
    const uint32_t p_hdr = fp4 && !mx ? 16u : 0u, p_row = mx ? 4u : 8u;
    const BufRsrc pb = make_buf(st.params, p_hdr + nbytes * p_row);
    const BufRsrc rb = make_buf(dense ? nullptr : st.rows, dense ? 0u : uint32_t(st.n) * 4u);
    // batches of kPvBatch 16-row slices: every load of a batch (staging, positions, scores)
    // goes out before any of it is used, so a batch costs one exposed round trip, not one per slice
    for (int32_t jb = a; jb < b; jb += 16 * kPvBatch) {
      wave_sync();                                        // the previous batch's staging is read
#pragma unroll
      for (int sb = 0; sb < kPvBatch; ++sb) {
        const int32_t j0 = jb + 16 * sb;
        if (j0 >= b) break;
        const int32_t jc = j0 + crow, jp = j0 + prow;
        const uint32_t co = jc < b ? (uint32_t(jc) * uint32_t(H) + uint32_t(h)) * (kAttnD / 2) + 16u * uint32_t(cq)
                                   : kOutOfRange;
        const uint32_t po = lane < 32 && jp < b && !(mx && (lane & 1))
                                ? p_hdr + (uint32_t(jp) * uint32_t(H) + uint32_t(h)) * p_row + 4u * uint32_t(lane & 1)
                                : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cb, (lds_ptr_t)&Sw[sb].codes[0][0], 16, co, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pb, (lds_ptr_t)&Sw[sb].params[0], 4, po, 0, 0, 0);
      }
      // this lane's tokens 4 kb + r of each slice (staged rows 4 r + kb): positions, then scores
      // (buffer loads with 32-bit offsets; a row past the range or of a dead head reads nothing
      // and gets p = 0 below)
      int32_t pos[kPvBatch][4];
#pragma unroll
      for (int sb = 0; sb < kPvBatch; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t j = jb + 16 * sb + 4 * r + kb;
          pos[sb][r] = dense ? j : int32_t(buf_ld32(rb, j < b ? uint32_t(j) * 4u : kOutOfRange, 0u));
        }
      float sv[kPvBatch][4];
#pragma unroll
      for (int sb = 0; sb < kPvBatch; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t j = jb + 16 * sb + 4 * r + kb;
          const uint32_t so = j < b && head_live ? (srow_off + uint32_t(pos[sb][r])) * 4u : kOutOfRange;
          sv[sb][r] = __uint_as_float(buf_ld32(sb_rsrc, so, 0u));
        }
      __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0): the staging has landed
      wave_sync();
#pragma unroll
      for (int sb = 0; sb < kPvBatch; ++sb) {
        if (jb + 16 * sb >= b) break;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t j = jb + 16 * sb + 4 * r + kb;
          p[r] = j < b && head_live ? __expf(sv[sb][r] - m) : 0.0f;
          if (l == 0) lsum += p[r];                       // the dense base lists every position once
        }
        const uint32_t pp01 = pack_f16x2(p[0], p[1]), pp23 = pack_f16x2(p[2], p[3]);
        const PvStage& S = Sw[sb];
        uint32_t d[4];
        uint2 vpw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * r + kb;
          const uint16_t* cr = reinterpret_cast<const uint16_t*>(&S.codes[row][0]);
          const uint32_t lo = cr[(16 * pv_chunk(row, n >> 3) + ((2 * n) & 15)) >> 1];
          const uint32_t hi = cr[(16 * pv_chunk(row, 2 + (n >> 3)) + ((2 * n) & 15)) >> 1];
          d[r] = lo | (hi << 16);
          vpw[r] = *reinterpret_cast<const uint2*>(&S.params[2 * row]);
        }
        if (fp4) {
          // FP4: A = e2m1 * block scale per element (exact in BF16), B = p (times the NVFP4
          // stream scale) in BF16, on the BF16 MFMA.  Tile mt's channel of this lane lies in
          // channel group g = mt / 4, block 4 g + n / 4 (NVFP4) or 2 g + n / 8 (MXFP4).
          const float gs = mx ? 1.0f : __uint_as_float(st.params[0]);
          short4_t bp;
#pragma unroll
          for (int r = 0; r < 4; ++r) bp[r] = short(__builtin_bit_cast(uint16_t, (__bf16)(p[r] * gs)));
          float sc[4][2];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (mx) {
              sc[r][0] = fp4_e8m0_value((vpw[r].x >> (8 * (n >> 3))) & 0xFFu);
              sc[r][1] = fp4_e8m0_value((vpw[r].x >> (8 * (2 + (n >> 3)))) & 0xFFu);
            } else {                                     // bytes n / 4 of both words, one conversion
              const uint32_t bsel = uint32_t(n >> 2);
              const fp4_f32x2 s2 = e4m3x2_value(__builtin_amdgcn_perm(vpw[r].y, vpw[r].x, bsel | ((4u + bsel) << 8)));
              sc[r][0] = s2.x;
              sc[r][1] = s2.y;
            }
          }
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const uint32_t bsel = uint32_t(mt >> 1);
            const uint32_t sel = bsel | ((4u + bsel) << 8) | 0x0C0C0000u;   // [x0.b, x1.b, 0, 0]
            uint32_t x01 = __builtin_amdgcn_perm(d[1], d[0], sel), x23 = __builtin_amdgcn_perm(d[3], d[2], sel);
            if (mt & 1) {                                  // high nibbles: one byte of two codes
              x01 = ((x01 >> 4) & 0x0Fu) | ((x01 >> 8) & 0xF0u);
              x23 = ((x23 >> 4) & 0x0Fu) | ((x23 >> 8) & 0xF0u);
            } else {
              x01 = (x01 & 0x0Fu) | ((x01 >> 4) & 0xF0u);
              x23 = (x23 & 0x0Fu) | ((x23 >> 4) & 0xF0u);
            }
            const fp4_f32x2 v01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x01, 1.0f, 0);
            const fp4_f32x2 v23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x23, 1.0f, 0);
            const int g = mt >> 2;
            short4_t av;
            av[0] = short(__builtin_bit_cast(uint16_t, (__bf16)(v01.x * sc[0][g])));
            av[1] = short(__builtin_bit_cast(uint16_t, (__bf16)(v01.y * sc[1][g])));
            av[2] = short(__builtin_bit_cast(uint16_t, (__bf16)(v23.x * sc[2][g])));
            av[3] = short(__builtin_bit_cast(uint16_t, (__bf16)(v23.y * sc[3][g])));
            o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bp, o[mt], 0, 0, 0);
          }
          continue;
        }
        f16x4_t bg[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const uint32_t w0 = g ? vpw[0].y : vpw[0].x, w1 = g ? vpw[1].y : vpw[1].x;
          const uint32_t w2 = g ? vpw[2].y : vpw[2].x, w3 = g ? vpw[3].y : vpw[3].x;
          const uint32_t s01 = __builtin_amdgcn_perm(w1, w0, 0x07060302u), s23 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
          const uint32_t m01 = __builtin_amdgcn_perm(w1, w0, 0x05040100u), m23 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
          const f16x2_t b01 = __builtin_bit_cast(f16x2_t, pp01) * __builtin_bit_cast(f16x2_t, s01);
          const f16x2_t b23 = __builtin_bit_cast(f16x2_t, pp23) * __builtin_bit_cast(f16x2_t, s23);
          bg[g] = f16x4_of(__builtin_bit_cast(uint32_t, b01), __builtin_bit_cast(uint32_t, b23));
          vmin[g] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pp01), __builtin_bit_cast(f16x2_t, m01), vmin[g], false);
          vmin[g] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pp23), __builtin_bit_cast(f16x2_t, m23), vmin[g], false);
          vmin[g] = __builtin_amdgcn_fdot2(b01, m1024, vmin[g], false);
          vmin[g] = __builtin_amdgcn_fdot2(b23, m1024, vmin[g], false);
        }
        // output tile mt takes nibble mt of each row's word, as binary16 1024 + code
        const uint32_t e0 = d[0] >> 4, e1 = d[1] >> 4, e2 = d[2] >> 4, e3 = d[3] >> 4;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const uint32_t bsel = uint32_t(mt >> 1);
          const uint32_t sel = bsel | 0x0C00u | ((4u + bsel) << 16) | 0x0C000000u;   // [x0.b, 0, x1.b, 0]
          const uint32_t x01 = (mt & 1) ? __builtin_amdgcn_perm(e1, e0, sel) : __builtin_amdgcn_perm(d[1], d[0], sel);
          const uint32_t x23 = (mt & 1) ? __builtin_amdgcn_perm(e3, e2, sel) : __builtin_amdgcn_perm(d[3], d[2], sel);
          const f16x4_t av = f16x4_of((x01 & nib) | 0x64006400u, (x23 & nib) | 0x64006400u);
          o[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bg[mt >> 2], o[mt], 0, 0, 0);
        }
      }
    }
  }

  // per head: the corrections and the probability sums over the 4 k-blocks
  float vm[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    vm[g] = vmin[g] + __shfl_xor(vmin[g], 16);
    vm[g] += __shfl_xor(vm[g], 32);
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  // merge the 4 waves (one reference maximum, so plain sums) through LDS
  __syncthreads();
  if (kb == 0) s_lds.merge.l[wave][n] = lsum;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_lds.merge.o[wave][n][pv_channel(mt, 4 * kb + i)] = o[mt][i] + vm[mt >> 2];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kAttnD; idx += kAThreads) {
    const int g = idx / kAttnD, ch = idx % kAttnD;
    float Ls = 0.0f, O = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kAWaves; ++wv) {
      Ls += s_lds.merge.l[wv][g];
      O += s_lds.merge.o[wv][g][ch];
    }
    const int64_t qi = int64_t(split) * Hq + h * G + g;
    if (ch == 0) {
      ws_ml[2 * qi] = block_max[qi];
      ws_ml[2 * qi + 1] = Ls;
    }
    ws_o[qi * kAttnD + ch] = O;
  }
}

// The two passes of one stream format; FP4 chains (FMT 1..4) of at most kSplitFp4Loops loops and
// without a tail.
template <int FMT, bool TL>
static hipError_t launch_split_fmt(const dim3& grid, const ChainArgs& kc, const ChainArgs& vc, int32_t T, int32_t H,
                                   int32_t G, const uint16_t* qp, float scale, int32_t wph, float* scores,
                                   float* block_max, float* ws_ml, float* ws_o, const uint16_t* kt,
                                   const uint16_t* vt, int32_t tail_len, hipStream_t stream) {
#define FLK_S(NLV)                                                                                         \
  case NLV:                                                                                                \
    hipLaunchKernelGGL((attn_scores_kernel<NLV, TL, FMT>), grid, dim3(kAThreads), 0, stream, kc, T, H, G, qp, \
                       scale, wph, scores, block_max, kt, tail_len);                                       \
    break;
#define FLK_P(NLV)                                                                                         \
  case NLV:                                                                                                \
    hipLaunchKernelGGL((attn_pv_kernel<NLV, FMT>), grid, dim3(kAThreads), 0, stream, vc, T, H, G, scores,    \
                       block_max, wph, ws_ml, ws_o, vt, tail_len);                                         \
    break;
  if constexpr (FMT == 0) {
    switch (kc.n_loops) {
      FLK_S(1) FLK_S(2) FLK_S(3) FLK_S(4) FLK_S(5) FLK_S(6) FLK_S(7) FLK_S(8)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (kc.n_loops) {
      FLK_S(1) FLK_S(2) FLK_S(3) FLK_S(4)
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (FMT == 0) {
    switch (vc.n_loops) {
      FLK_P(1) FLK_P(2) FLK_P(3) FLK_P(4) FLK_P(5) FLK_P(6) FLK_P(7) FLK_P(8)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (vc.n_loops) {
      FLK_P(1) FLK_P(2) FLK_P(3) FLK_P(4)
      default: return hipErrorInvalidValue;
    }
  }
#undef FLK_P
#undef FLK_S
  return hipGetLastError();
}

hipError_t launch_attn_split(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                             const ChainArgs& vc, const void* k_tail, const void* v_tail, int32_t tail_len,
                             float scale, int32_t wph, int32_t splits, float* scores, float* block_max, float* ws_ml,
                             float* ws_o, hipStream_t stream) {
  const uint16_t* kt = static_cast<const uint16_t*>(k_tail);
  const uint16_t* vt = static_cast<const uint16_t*>(v_tail);
  const int32_t G = Hq / H;
  const dim3 grid(static_cast<unsigned>(splits), static_cast<unsigned>(H));
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  if (fmt != 0 && (tail_len > 0 || kc.n_loops > kSplitFp4Loops || vc.n_loops > kSplitFp4Loops))
    return hipErrorInvalidValue;
#define FLK_F(F, TL)                                                                                       \
  case F:                                                                                                  \
    return launch_split_fmt<F, TL>(grid, kc, vc, T, H, G, qp, scale, wph, scores, block_max, ws_ml, ws_o, kt, vt, \
                                   tail_len, stream);
  if (tail_len > 0) return launch_split_fmt<0, true>(grid, kc, vc, T, H, G, qp, scale, wph, scores, block_max, ws_ml,
                                                     ws_o, kt, vt, tail_len, stream);
  switch (fmt) {
    FLK_F(0, false) FLK_F(1, false) FLK_F(2, false) FLK_F(3, false) FLK_F(4, false)
    default: return hipErrorInvalidValue;
  }
#undef FLK_F
}

}  // namespace flk
