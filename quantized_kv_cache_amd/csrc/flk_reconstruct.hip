// flk_reconstruct.hip -- gfx950 reconstruction of X_hat[R] from a packed loop chain.
//
// One pass over the logical tensor, each output element written once with a 16-byte
// streaming store.  A block owns a 64-token tile of a strip of up to 512 channels of the
// flattened H*D axis.  Each wave walks whole tokens (64 lanes x 8 channels when the strip
// is 512 channels wide), so whether a compact loop lists a token is uniform across the wave
// and absent positions cost no arithmetic.  Per compact loop the block finds the tile's
// compact rows with a parallel lower_bound and an LDS position -> row table; K params
// (one per channel and 64 compact rows, or per tile with tile groups) are staged in LDS as
// binary32 pairs.  Each element
// walks base -> delta2 -> ... with the encoder's BF16 rounding after every step
// (FlashLoop RFC, vllm-rlt #156, section 3.3: t1 reads base + delta2, t2 adds delta3, t4
// adds delta4; an absent residual means inheritance).
#include "flk_device.h"
#include "flk_internal.h"

namespace flk {

#ifndef FLK_RECON_BATCH
#define FLK_RECON_BATCH 4
#endif
constexpr int kRThreads = 256;
constexpr int kTile = 64;                 // tokens per block, narrow rows
constexpr int kBatch = FLK_RECON_BATCH;   // tokens whose loads a wave issues together
#ifndef FLK_RECON_TPW
#define FLK_RECON_TPW 4
#endif
constexpr int kWideTokPerWave = FLK_RECON_TPW;  // tokens per wave, wide rows (divides 64)
constexpr int kMaxStripCh = 512;

template <int KIND, int NL>
__global__ __launch_bounds__(kRThreads) void reconstruct_kernel(ChainArgs chain, int32_t T,
                                                                 int32_t H, int32_t D,
                                                                 int32_t lpt_log2,
                                                                 uint16_t* __restrict__ out) {
  __shared__ int32_t s_map[NL][kTile];
  __shared__ int32_t s_rg0[NL];
  __shared__ __align__(16) float2 s_kp[KIND == FLK_KIND_K ? NL : 1][2][KIND == FLK_KIND_K ? kMaxStripCh : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lpt = 1 << lpt_log2;               // lanes per token (chunks of 8 channels)
  const int32_t W = H * D;
  const int32_t cpr = W >> 3;
  const int cl = lane & (lpt - 1);
  const int32_t chunk = int32_t(blockIdx.y) * lpt + cl;
  const bool cact = chunk < cpr;
  const int64_t ch = int64_t(chunk) * 8;
  const int32_t strip_ch0 = int32_t(blockIdx.y) * lpt * 8;
  const int32_t t0 = int32_t(blockIdx.x) * kTile;

  // ---- per-tile tables: compact row of each position, and K params of the touched groups
  for (int idx = tid; idx < NL * kTile; idx += kRThreads) s_map[idx / kTile][idx % kTile] = -1;
  __syncthreads();
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const StreamArgs st = chain.s[l];
    int32_t rg0 = int32_t(blockIdx.x), nrg = 1;
    if (st.rows != nullptr) {
      const int32_t lo = block_lower_bound(st.rows, st.n, t0);
      int found = 0;
      if (tid < kTile) {
        const int32_t j = lo + tid;
        if (j < st.n) {
          const int32_t p = st.rows[j];
          if (p >= t0 && p < t0 + kTile) { s_map[l][p - t0] = j; found = 1; }
        }
      }
      const int32_t cnt = __syncthreads_count(found);
      // the rowgroups holding the tile's rows (at most 2), or with tile groups the tile's own
      rg0 = chain.ktile ? int32_t(blockIdx.x) : lo / kGroup;
      nrg = cnt == 0 ? 0 : chain.ktile ? 1 : ((lo + cnt - 1) / kGroup - rg0 + 1);
    }
    if (KIND == FLK_KIND_K) {
      // stage (min, scale) of rowgroups rg0 .. rg0 + nrg - 1 (at most 2) for this strip
      for (int idx = tid; idx < nrg * kMaxStripCh; idx += kRThreads) {
        const int slot = idx / kMaxStripCh, c = idx % kMaxStripCh;
        if (strip_ch0 + c < W && c < lpt * 8) {
          const uint32_t pw = st.params[int64_t(rg0 + slot) * W + strip_ch0 + c];
          s_kp[l][slot][c] = make_float2(f16_bits_to_f32(pw & 0xFFFFu), f16_bits_to_f32(pw >> 16));
        }
      }
      if (tid == 0) s_rg0[l] = rg0;
    }
  }
  __syncthreads();
  if (!cact) return;

  // V: the lane's head and group within the head are fixed.
  const int32_t S = (D + kGroup - 1) / kGroup;
  const int32_t vh = int32_t(ch / D);
  const int32_t vg = int32_t((ch - int64_t(vh) * D) / kGroup);

  const int tpw = 64 >> lpt_log2;              // tokens per wave step
  const int tslot = lane >> lpt_log2;
  const int steps = kTile / (4 * tpw);         // token steps per wave
  for (int k0 = 0; k0 < steps; k0 += 4) {
    uint32_t cw[4][NL];
    uint32_t vp[4][NL];
    int32_t jj[4][NL];
    // phase A: issue every load of 4 tokens x NL loops
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t tl = (wave + 4 * (k0 + i)) * tpw + tslot;   // token within the tile
      const int32_t t = t0 + tl;
      const bool ok = (k0 + i) < steps && t < T;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const StreamArgs st = chain.s[l];
        int32_t j = ok ? (st.rows == nullptr ? t : s_map[l][tl]) : -1;
        jj[i][l] = j;
        cw[i][l] = 0;
        vp[i][l] = 0;
        if (j >= 0) {
          cw[i][l] = ld_stream32(st.codes + ((int64_t(j) * W + ch) >> 1));
          if (KIND == FLK_KIND_V) vp[i][l] = st.params[(int64_t(j) * H + vh) * S + vg];
        }
      }
    }
    // phase B: decode and accumulate in loop order, store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (jj[i][0] < 0) continue;
      const int32_t tl = (wave + 4 * (k0 + i)) * tpw + tslot;
      float acc[8];
      uint4 packed = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const int32_t j = jj[i][l];
        if (j < 0) continue;
        float c[8], m[8], s[8];
        codes8_to_f32(cw[i][l], c);
        if (KIND == FLK_KIND_K) {
          const int slot = chain.ktile ? 0 : (j >> 6) - s_rg0[l];
          const float4* kp = reinterpret_cast<const float4*>(&s_kp[l][slot][cl * 8]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float4 q = kp[e];
            m[2 * e] = q.x; s[2 * e] = q.y; m[2 * e + 1] = q.z; s[2 * e + 1] = q.w;
          }
        } else {
          const float mm = f16_bits_to_f32(vp[i][l] & 0xFFFFu), ss = f16_bits_to_f32(vp[i][l] >> 16);
#pragma unroll
          for (int e = 0; e < 8; ++e) { m[e] = mm; s[e] = ss; }
        }
        float d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = decode(c[e], m[e], s[e]);
        if (l == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = d[e];
          packed = round_bf16x8(acc);
        } else {
          round_bf16x8(d);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = acc[e] + d[e];
          packed = round_bf16x8(acc);
        }
      }
      st_stream(out + int64_t(t0 + tl) * W + ch, packed);
    }
  }
}

// Wide rows (H*D >= 512 channels): a strip is 512 channels, 64 lanes x 8 channels, and every
// wave works alone on kWideTokPerWave consecutive tokens with no block barrier.  It reads its
// tile's slice of each compact loop's tile index, scatters those rows into a wave-private LDS
// table indexed by position, and then reconstructs one token at a time, so a token's compact
// row is a scalar (readlane) and every access is a buffer access with a scalar row offset.
// Many short waves keep more loads in flight than a few long ones.  A token that a compact
// loop does not list loads row 0 (a cache hit) and skips that loop's arithmetic: its value is
// inherited bit for bit.  Params stay packed FP16 pairs and feed v_fma_mix_f32 directly.
// SPARSE has bit l set when loop l is compact; with RT the pattern is read from the chain at
// run time instead (chains longer than 4 loops).
template <int KIND, int NL, uint32_t SPARSE, bool RT>
__device__ __forceinline__ void reconstruct_wide_body(const ChainArgs& chain, int32_t T, int32_t H, int32_t D,
                                                      uint16_t* __restrict__ out, uint32_t bx, uint32_t by) {
  constexpr int kTokPerWave = kWideTokPerWave;
  __shared__ int32_t s_map[kRThreads / 64][NL][kTokPerWave];
  auto is_sparse = [&](int l) -> bool {
    return RT ? chain.s[l].rows != nullptr : ((SPARSE >> l) & 1u) != 0;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int32_t W = H * D;
  const int32_t chunk = int32_t(by) * 64 + lane;
  const int32_t ch = chunk * 8;
  const int32_t tw = int32_t(bx) * (kTokPerWave * (kRThreads / 64)) + wave * kTokPerWave;
  if (tw >= T) return;                                   // wave-uniform, no barrier follows

  // ---- this wave's position -> compact row table (wave-private; no block barrier) ----
  // The tile index gives the compact rows of the wave's 64-position tile; lane L looks at
  // the tile's L-th compact row and records it if it falls in the wave's own positions.
  const int32_t tile = tw / kGroup;
  int32_t lo[NL], hi[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    lo[l] = is_sparse(l) ? uniform(chain.s[l].tile_start[tile]) : 0;
    hi[l] = is_sparse(l) ? uniform(chain.s[l].tile_start[tile + 1]) : 0;
    if (is_sparse(l) && lane < kTokPerWave) s_map[wave][l][lane] = -1;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (!is_sparse(l)) continue;
    const int32_t j = lo[l] + lane;
    if (j < hi[l]) {
      const uint32_t o = uint32_t(chain.s[l].rows[j] - tw);
      if (o < uint32_t(kTokPerWave)) s_map[wave][l][o] = j;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int32_t mapv[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) mapv[l] = is_sparse(l) ? s_map[wave][l][lane & (kTokPerWave - 1)] : 0;
  if (chunk >= (W >> 3)) return;

  const int32_t S = (D + kGroup - 1) / kGroup;
  const int32_t vh = ch / D;
  const uint32_t v_voff = uint32_t(vh * S + (ch - vh * D) / kGroup) * 4u;  // V param within a row
  const uint32_t vrow_bytes = uint32_t(H * S) * 4u;
  const uint32_t krow_bytes = uint32_t(W) * 4u;        // one K rowgroup of params
  const uint32_t k_voff = uint32_t(ch) * 4u;
  const uint32_t crow_bytes = uint32_t(W) >> 1;
  const uint32_t c_voff = uint32_t(ch) >> 1;
  BufRsrc crs[NL], prs[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const uint32_t n = uint32_t(chain.s[l].n);
    crs[l] = make_buf(chain.s[l].codes, n * crow_bytes);
    const uint32_t krows = chain.ktile ? (uint32_t(T) + kGroup - 1) / kGroup : (n + kGroup - 1) / kGroup;
    prs[l] = make_buf(chain.s[l].params, KIND == FLK_KIND_K ? krows * krow_bytes : n * vrow_bytes);
  }
  const BufRsrc ors = make_buf(out, uint32_t(T) * uint32_t(W) * 2u);
  const uint32_t o_voff = uint32_t(ch) * 2u;
  const uint32_t orow_bytes = uint32_t(W) * 2u;

  // K params: one resident rowgroup per loop.  A dense loop's tokens lie in one rowgroup;
  // a compact loop's rows for them span at most two, so the set is reloaded at most once.
  // With tile groups every loop's parameter row is the tile's own.
  uint4 kreg[NL][2];
  int32_t krg[NL];
  if (KIND == FLK_KIND_K) {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      krg[l] = chain.ktile ? tile : (is_sparse(l) ? lo[l] : tw) / kGroup;
      const uint32_t soff = uint32_t(krg[l]) * krow_bytes;
      kreg[l][0] = buf_ld128(prs[l], k_voff, soff);
      kreg[l][1] = buf_ld128(prs[l], k_voff + 16u, soff);
    }
  }

  // Software pipeline over batches of kBatch tokens: batch b+1's loads are issued before
  // batch b's stores.  A token a compact loop does not list loads row 0 (a cache hit) and
  // skips that loop's arithmetic.
  constexpr int kBatches = kTokPerWave / kBatch;
  uint32_t cw[2][kBatch][NL], vp[2][kBatch][NL];
  int32_t jj[2][kBatch][NL];
  auto issue = [&](int b, int buf) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int32_t t = tw + b * kBatch + i;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        int32_t j = is_sparse(l) ? __builtin_amdgcn_readlane(mapv[l], b * kBatch + i) : t;
        if (t >= T) j = -1;
        jj[buf][i][l] = j;
        const uint32_t row = uint32_t(max(j, 0));
        cw[buf][i][l] = buf_ld32<kCacheStream>(crs[l], c_voff, row * crow_bytes);
        if (KIND == FLK_KIND_V) vp[buf][i][l] = buf_ld32(prs[l], v_voff, row * vrow_bytes);
      }
    }
  };
  issue(0, 0);
#pragma unroll
  for (int b = 0; b < kBatches; ++b) {
    const int cur = b & 1;
    if (b + 1 < kBatches) issue(b + 1, cur ^ 1);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (jj[cur][i][0] < 0) continue;
      const int32_t t = tw + b * kBatch + i;
      float acc[8];
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const int32_t j = jj[cur][i][l];
        if (j < 0) continue;
        float c[8];
        codes8_to_f32(cw[cur][i][l], c);
        uint32_t pw[8];
        if (KIND == FLK_KIND_K) {
          if (is_sparse(l) && !chain.ktile && (j / kGroup) != krg[l]) {   // crossed into the next rowgroup
            krg[l] = j / kGroup;
            const uint32_t soff = uint32_t(krg[l]) * krow_bytes;
            kreg[l][0] = buf_ld128(prs[l], k_voff, soff);
            kreg[l][1] = buf_ld128(prs[l], k_voff + 16u, soff);
          }
          const uint4 a = kreg[l][0], bq = kreg[l][1];
          pw[0] = a.x; pw[1] = a.y; pw[2] = a.z; pw[3] = a.w;
          pw[4] = bq.x; pw[5] = bq.y; pw[6] = bq.z; pw[7] = bq.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pw[e] = vp[cur][i][l];
        }
        float d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          d[e] = decode(c[e], f16_bits_to_f32(pw[e] & 0xFFFFu), f16_bits_to_f32(pw[e] >> 16));
        round_bf16x8_inplace(d);
        if (l == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = d[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = round_bf16(acc[e] + d[e]);
        }
      }
      buf_st128<kCacheStream>(pack_exact_bf16x8(acc), ors, o_voff, uint32_t(t) * orow_bytes);
    }
  }
}

template <int KIND, int NL, uint32_t SPARSE, bool RT>
__global__ __launch_bounds__(kRThreads) void reconstruct_wide_kernel(ChainArgs chain, int32_t T, int32_t H,
                                                                      int32_t D, uint16_t* __restrict__ out) {
  uint32_t bx, by;
  xcd_block(bx, by);                                     // the 4 blocks of a tile share K params
  reconstruct_wide_body<KIND, NL, SPARSE, RT>(chain, T, H, D, out, bx, by);
}

template <int KIND>
static void launch_kind(dim3 grid, const ChainArgs& chain, int32_t T, int32_t H, int32_t D,
                        int32_t lpt_log2, uint16_t* out, hipStream_t stream) {
  if (lpt_log2 == 6) {
    constexpr int kTokPerBlock = kWideTokPerWave * (kRThreads / 64);
    const dim3 wgrid(unsigned((T + kTokPerBlock - 1) / kTokPerBlock), grid.y);
    uint32_t mask = 0;
    for (int l = 0; l < chain.n_loops; ++l) mask |= (chain.s[l].rows != nullptr ? 1u : 0u) << l;
#define FLK_W(NLV, M)                                                                              \
  if (chain.n_loops == NLV && mask == M) {                                                         \
    hipLaunchKernelGGL((reconstruct_wide_kernel<KIND, NLV, M, false>), wgrid, dim3(kRThreads), 0,  \
                       stream, chain, T, H, D, out);                                               \
    return;                                                                                        \
  }
    FLK_W(1, 0)
    FLK_W(2, 0) FLK_W(2, 2)
    FLK_W(3, 0) FLK_W(3, 2) FLK_W(3, 4) FLK_W(3, 6)
    FLK_W(4, 0) FLK_W(4, 2) FLK_W(4, 4) FLK_W(4, 6) FLK_W(4, 8) FLK_W(4, 10) FLK_W(4, 12) FLK_W(4, 14)
#undef FLK_W
#define FLK_W(NLV)                                                                                 \
  case NLV:                                                                                        \
    hipLaunchKernelGGL((reconstruct_wide_kernel<KIND, NLV, 0, true>), wgrid, dim3(kRThreads), 0,   \
                       stream, chain, T, H, D, out);                                               \
    break;
    switch (chain.n_loops) {
      FLK_W(5) FLK_W(6) FLK_W(7) FLK_W(8)
      default: break;
    }
#undef FLK_W
    return;
  }
#define FLK_R(NLV)                                                                             \
  case NLV:                                                                                    \
    hipLaunchKernelGGL((reconstruct_kernel<KIND, NLV>), grid, dim3(kRThreads), 0, stream, chain, \
                       T, H, D, lpt_log2, out);                                                \
    break;
  switch (chain.n_loops) {
    FLK_R(1) FLK_R(2) FLK_R(3) FLK_R(4) FLK_R(5) FLK_R(6) FLK_R(7) FLK_R(8)
    default: break;
  }
#undef FLK_R
}

hipError_t launch_reconstruct(int kind, int32_t T, int32_t H, int32_t D, const ChainArgs& chain,
                              void* out, hipStream_t stream) {
  const int32_t cpr = H * D / 8;
  int lpt_log2 = 3;
  while ((1 << lpt_log2) < cpr && lpt_log2 < 6) ++lpt_log2;
  const int lpt = 1 << lpt_log2;
  const dim3 grid(unsigned((T + kTile - 1) / kTile), unsigned((cpr + lpt - 1) / lpt));
  uint16_t* o = static_cast<uint16_t*>(out);
  if (kind == FLK_KIND_K) launch_kind<FLK_KIND_K>(grid, chain, T, H, D, lpt_log2, o, stream);
  else launch_kind<FLK_KIND_V>(grid, chain, T, H, D, lpt_log2, o, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Batched reconstruct: one launch rebuilds up to kRecBatch tensors (K and V mixed) whose chains
// share the loop count and compact pattern, all with rows of at least 512 channels.  Blocks are
// numbered unit after unit (in XCD order, as above) and each runs its unit's kind of body.
// ---------------------------------------------------------------------------------------
struct RecUnit {
  ChainArgs c;
  uint16_t* out;
  int32_t T, H, D, kind;
  uint32_t gx, block0;
};
struct RecBatch {
  RecUnit u[kRecBatch];
  int32_t n_units;
};

static_assert(sizeof(RecBatch) <= 4096, "a batch travels as kernel arguments (4 KiB at most)");

template <int NL, uint32_t SPARSE, bool RT>
__global__ __launch_bounds__(kRThreads) void reconstruct_batch_kernel(RecBatch b) {
  const uint32_t lin = xcd_remap(blockIdx.x, gridDim.x);
  int ui = 0;
#pragma unroll
  for (int i = 1; i < kRecBatch; ++i)
    if (i < b.n_units && lin >= b.u[i].block0) ui = i;
  const RecUnit& u = b.u[ui];
  const uint32_t lb = lin - u.block0;
  const uint32_t by = lb / u.gx, bx = lb - by * u.gx;
  if (u.kind == FLK_KIND_K) reconstruct_wide_body<FLK_KIND_K, NL, SPARSE, RT>(u.c, u.T, u.H, u.D, u.out, bx, by);
  else reconstruct_wide_body<FLK_KIND_V, NL, SPARSE, RT>(u.c, u.T, u.H, u.D, u.out, bx, by);
}

static uint32_t chain_mask(const ChainArgs& c) {
  uint32_t m = 0;
  for (int l = 0; l < c.n_loops; ++l) m |= (c.s[l].rows != nullptr ? 1u : 0u) << l;
  return m;
}

bool reconstruct_batchable(int32_t H, int32_t D) { return H * D >= 512; }

static hipError_t launch_rec_batch(const RecBatch& b, uint32_t blocks, int nl, uint32_t mask, hipStream_t stream) {
#define FLK_RB(NLV, M)                                                                                 \
  if (nl == NLV && mask == M) {                                                                        \
    hipLaunchKernelGGL((reconstruct_batch_kernel<NLV, M, false>), dim3(blocks), dim3(kRThreads), 0, stream, b); \
    return hipGetLastError();                                                                          \
  }
  FLK_RB(1, 0)
  FLK_RB(2, 0) FLK_RB(2, 2)
  FLK_RB(3, 0) FLK_RB(3, 2) FLK_RB(3, 4) FLK_RB(3, 6)
  FLK_RB(4, 0) FLK_RB(4, 2) FLK_RB(4, 4) FLK_RB(4, 6) FLK_RB(4, 8) FLK_RB(4, 10) FLK_RB(4, 12) FLK_RB(4, 14)
#undef FLK_RB
#define FLK_RB(NLV)                                                                                    \
  case NLV:                                                                                            \
    hipLaunchKernelGGL((reconstruct_batch_kernel<NLV, 0, true>), dim3(blocks), dim3(kRThreads), 0, stream, b); \
    return hipGetLastError();
  switch (nl) {
    FLK_RB(5) FLK_RB(6) FLK_RB(7) FLK_RB(8)
    default: return hipErrorInvalidValue;
  }
#undef FLK_RB
}

hipError_t launch_reconstruct_batch(const RecArgs* units, int n_units, hipStream_t stream) {
  constexpr int kTokPerBlock = kWideTokPerWave * (kRThreads / 64);
  int i = 0;
  while (i < n_units) {
    // a run of units with the same loop count and compact pattern, at most kRecBatch long
    const int nl = units[i].chain.n_loops;
    const uint32_t mask = chain_mask(units[i].chain);
    RecBatch b{};
    uint32_t blocks = 0;
    while (i < n_units && b.n_units < kRecBatch && units[i].chain.n_loops == nl &&
           chain_mask(units[i].chain) == mask) {
      const RecArgs& a = units[i];
      RecUnit& r = b.u[b.n_units++];
      r.c = a.chain;
      r.out = static_cast<uint16_t*>(a.out);
      r.T = a.T;
      r.H = a.H;
      r.D = a.D;
      r.kind = a.kind;
      r.gx = uint32_t((a.T + kTokPerBlock - 1) / kTokPerBlock);
      r.block0 = blocks;
      blocks += r.gx * uint32_t((a.H * a.D / 8 + 63) / 64);
      ++i;
    }
    const hipError_t e = launch_rec_batch(b, blocks, nl, mask, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace flk
