// flk_attn.hip -- single-token grouped-query decode attention read straight from packed
// K/V chains (FlashLoop RFC, vllm-rlt #156, section 3.3: optimized readers consume packed
// base/residual tiles during QK/PV instead of keeping a BF16 shadow cache).
//
// Split-token scheme: block (split, h) walks the 64-token tiles of its token range for KV
// head h, decodes K_hat and V_hat of each tile into LDS with the same chain reader the
// reconstruct kernel uses, scores the G = Hq/H query heads of the group, and keeps an
// online softmax (running max m, mass l, weighted values o) per query head in binary32.
// A second kernel merges the per-split (m, l, o) triples.
#include "flk_chain.h"

namespace flk {

constexpr int kAThreads = 256;
constexpr int kAttnD = 128;
constexpr int kSplitTiles = 16;             // 1024 tokens per split
constexpr int kMaxG = 16;

static int32_t n_splits(int32_t T) {
  const int32_t tiles = (T + kGroup - 1) / kGroup;
  return (tiles + kSplitTiles - 1) / kSplitTiles;
}

size_t attn_workspace_bytes(int32_t T, int32_t H, int32_t Hq) {
  (void)H;
  return size_t(n_splits(T)) * size_t(Hq) * (2 + kAttnD) * sizeof(float);
}

__global__ __launch_bounds__(kAThreads) void attn_partial_kernel(
    ChainArgs kc, ChainArgs vc, int32_t T, int32_t H, int32_t G, const uint16_t* __restrict__ q,
    float scale, float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  __shared__ int32_t s_mapk[FLK_MAX_LOOPS][kGroup];
  __shared__ int32_t s_mapv[FLK_MAX_LOOPS][kGroup];
  // decoded tiles are exactly BF16, so they are staged as BF16 bit patterns
  __shared__ uint16_t sK[kGroup][kAttnD + 2];
  __shared__ uint16_t sV[kGroup][kAttnD + 2];
  __shared__ float sQ[kMaxG][kAttnD];
  __shared__ float sP[kMaxG][kGroup];
  __shared__ float sScale[kMaxG];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cc = tid & 15;
  const int rs = tid >> 4;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int Hq = H * G;
  const int64_t ch = int64_t(h) * kAttnD + cc * 8;

  for (int idx = tid; idx < G * kAttnD; idx += kAThreads)
    sQ[idx / kAttnD][idx % kAttnD] = bf16_to_f32(q[int64_t(h * G + idx / kAttnD) * kAttnD + idx % kAttnD]);

  // per query head running state: wave w owns heads w, w+4, ...; lane owns channels 2*lane, 2*lane+1
  float m_run[kMaxG / 4], l_run[kMaxG / 4], o_run[kMaxG / 4][2];
#pragma unroll
  for (int a = 0; a < kMaxG / 4; ++a) { m_run[a] = -__builtin_inff(); l_run[a] = 0.0f; o_run[a][0] = o_run[a][1] = 0.0f; }

  const int32_t tile0 = split * kSplitTiles;
  const int32_t tiles = (T + kGroup - 1) / kGroup;
  const int32_t tile1 = min(tiles, tile0 + kSplitTiles);
  for (int32_t tile = tile0; tile < tile1; ++tile) {
    build_tile_maps(kc, tile * kGroup, s_mapk);
    build_tile_maps(vc, tile * kGroup, s_mapv);
    float acc[4][8];
    bool tact[4];
    read_chain_tile<FLK_KIND_K>(kc, tile, T, H, kAttnD, ch, rs, s_mapk, acc, tact);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) sK[rs + 16 * i][cc * 8 + e] = uint16_t(__float_as_uint(acc[i][e]) >> 16);
    read_chain_tile<FLK_KIND_V>(vc, tile, T, H, kAttnD, ch, rs, s_mapv, acc, tact);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) sV[rs + 16 * i][cc * 8 + e] = uint16_t(__float_as_uint(acc[i][e]) >> 16);
    __syncthreads();

    // scores: wave w, heads g = w, w+4, ...; lane = token within the tile
    const bool valid = tile * kGroup + lane < T;
#pragma unroll
    for (int a = 0; a < kMaxG / 4; ++a) {
      const int g = wave + 4 * a;
      if (g >= G) break;
      float sc = 0.0f;
      for (int c = 0; c < kAttnD; ++c) sc = __builtin_fmaf(sQ[g][c], bf16_to_f32(sK[lane][c]), sc);
      sc = valid ? sc * scale : -__builtin_inff();
      float mt = sc;
      for (int off = 32; off > 0; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
      const float m_new = fmaxf(m_run[a], mt);
      const float p = valid ? __expf(sc - m_new) : 0.0f;
      float ps = p;
      for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
      const float corr = __expf(m_run[a] - m_new);
      l_run[a] = l_run[a] * corr + ps;
      m_run[a] = m_new;
      sP[g][lane] = p;
      if (lane == 0) sScale[g] = corr;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < kMaxG / 4; ++a) {
      const int g = wave + 4 * a;
      if (g >= G) break;
      float o0 = o_run[a][0] * sScale[g], o1 = o_run[a][1] * sScale[g];
      for (int t = 0; t < kGroup; ++t) {
        const float p = sP[g][t];
        o0 = __builtin_fmaf(p, bf16_to_f32(sV[t][2 * lane]), o0);
        o1 = __builtin_fmaf(p, bf16_to_f32(sV[t][2 * lane + 1]), o1);
      }
      o_run[a][0] = o0;
      o_run[a][1] = o1;
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < kMaxG / 4; ++a) {
    const int g = wave + 4 * a;
    if (g >= G) break;
    const int64_t qi = int64_t(split) * Hq + h * G + g;
    if (lane == 0) { ws_ml[2 * qi] = m_run[a]; ws_ml[2 * qi + 1] = l_run[a]; }
    ws_o[qi * kAttnD + 2 * lane] = o_run[a][0];
    ws_o[qi * kAttnD + 2 * lane + 1] = o_run[a][1];
  }
}

__global__ __launch_bounds__(kAttnD) void attn_combine_kernel(int32_t splits, int32_t Hq,
                                                              const float* __restrict__ ws_ml,
                                                              const float* __restrict__ ws_o,
                                                              uint16_t* __restrict__ out) {
  const int i = blockIdx.x;
  const int c = threadIdx.x;
  float M = -__builtin_inff();
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ws_ml[2 * (int64_t(s) * Hq + i)]);
  float L = 0.0f, O = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const int64_t qi = int64_t(s) * Hq + i;
    const float w = __expf(ws_ml[2 * qi] - M);
    L = __builtin_fmaf(ws_ml[2 * qi + 1], w, L);
    O = __builtin_fmaf(ws_o[qi * kAttnD + c], w, O);
  }
  out[int64_t(i) * kAttnD + c] = __builtin_bit_cast(uint16_t, (__bf16)(O / L));
}

hipError_t launch_decode_attn(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, float scale, void* out,
                              void* ws, hipStream_t stream) {
  (void)D;
  const int32_t splits = n_splits(T);
  const int32_t G = Hq / H;
  float* ws_ml = static_cast<float*>(ws);
  float* ws_o = ws_ml + size_t(splits) * Hq * 2;
  hipLaunchKernelGGL(attn_partial_kernel, dim3(splits, H), dim3(kAThreads), 0, stream, kc, vc, T,
                     H, G, static_cast<const uint16_t*>(q), scale, ws_ml, ws_o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(Hq), dim3(kAttnD), 0, stream, splits, Hq, ws_ml,
                     ws_o, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace flk
