// flk_attn.hip -- single-token grouped-query decode attention read straight from packed K/V
// chains (FlashLoop RFC, vllm-rlt #156, section 3.3: optimized readers consume the packed
// base/residual tiles during QK and PV instead of keeping a BF16 shadow cache).
//
// A block owns one KV head and a run of 64-token tiles.  For each tile it
//   1. decodes K_hat and V_hat of the tile into LDS, bit for bit as the encoder left them:
//      the leading dense loops accumulate in registers (one thread per token x 8 channels),
//      every later loop reads only the rows it lists (compact rows of the tile, found with the
//      tile index) and updates LDS in place, so an absent token costs nothing;
//   2. computes the G query heads' scores for its 64 tokens with MFMA, as S^T = K_hat Q^T
//      (v_mfma_f32_16x16x32_bf16, one 16-token slice per wave);
//   3. keeps an online softmax per (wave, query head) in binary32 and accumulates
//      O^T += V_hat^T P^T with v_mfma_f32_16x16x16_bf16 -- the score tile's register layout is
//      exactly the P^T operand's, so probabilities never leave registers.
// At the end the 4 waves' (m, l, O) merge through LDS into one partial per (block, query head);
// a second kernel merges the partials of all blocks.
#include "flk_device.h"
#include "flk_internal.h"

namespace flk {

constexpr int kAThreads = 256;
constexpr int kAttnD = 128;
constexpr int kMaxG = 16;
constexpr int kLdsRow = kAttnD + 8;         // BF16 per LDS row: 272 bytes keep MFMA reads conflict-free
#ifndef FLK_ATTN_BLOCKS
#define FLK_ATTN_BLOCKS 2048
#endif
constexpr int kAttnBlocks = FLK_ATTN_BLOCKS;  // aim for about this many blocks per launch

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

static int32_t tiles_per_split(int32_t T, int32_t H) {
  const int64_t tiles = (int64_t(T) + kGroup - 1) / kGroup;
  const int64_t per = (tiles * H + kAttnBlocks - 1) / kAttnBlocks;
  return int32_t(per < 1 ? 1 : per);
}
static int32_t n_splits(int32_t T, int32_t H) {
  const int32_t tiles = (T + kGroup - 1) / kGroup;
  const int32_t tps = tiles_per_split(T, H);
  return (tiles + tps - 1) / tps;
}

size_t attn_workspace_bytes(int32_t T, int32_t H, int32_t Hq) {
  return size_t(n_splits(T, H)) * size_t(Hq) * (2 + kAttnD) * sizeof(float);
}

// Decode loop l's 8 channels of one item into d[] (binary32 values that are exactly BF16).
// K: params of the 8 channels come from the LDS copy of the item's parameter row; V: one
// parameter for the item's 64-channel group.
__device__ __forceinline__ void decode_item(uint32_t cw, const uint32_t p[8], float d[8]) {
  float c[8];
  codes8_to_f32(cw, c);
#pragma unroll
  for (int e = 0; e < 8; ++e) d[e] = decode(c[e], f16_bits_to_f32(p[e] & 0xFFFFu), f16_bits_to_f32(p[e] >> 16));
  round_bf16x8_inplace(d);
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

// Decode one chain's tile (64 tokens from t0, KV head h, all 128 channels) into s[64][kLdsRow].
// Thread (ts = tid >> 4, oc = tid & 15) owns channels 8*oc..8*oc+7 of tokens ts + 16*i.
// kp is LDS scratch for K parameter rows: [NL][2][128].  Contains barriers; all threads call.
template <int KIND, int NL>
__device__ __forceinline__ void decode_tile(const ChainArgs& c, int32_t tile, int32_t T, int32_t H,
                                            int32_t h, uint16_t (*s)[kLdsRow], uint32_t (*kp)[2][kAttnD]) {
  const int tid = threadIdx.x;
  const int oc = tid & 15, ts = tid >> 4;
  const int32_t t0 = tile * kGroup;
  const int nl = c.n_loops;

  // compact row range of every loop for this tile (dense loops: the tile's positions)
  int32_t lo[NL], hi[NL];
  bool dense[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    dense[l] = l >= nl || c.s[l].rows == nullptr;
    lo[l] = dense[l] ? t0 : uniform(c.s[l].tile_start[tile]);
    hi[l] = dense[l] ? min(t0 + kGroup, T) : uniform(c.s[l].tile_start[tile + 1]);
  }
  int dp = 0;                                             // leading dense loops
#pragma unroll
  for (int l = 0; l < NL; ++l)
    if (l < nl && dense[l] && dp == l) dp = l + 1;

  // K: stage the parameter rows the tile needs (rowgroups lo/64 and lo/64 + 1 per loop)
  if (KIND == FLK_KIND_K) {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (l >= nl) continue;
      const int32_t rg = lo[l] / kGroup + (tid >> 7);     // a dense loop needs only the first
      const int32_t nrg = (c.s[l].n + kGroup - 1) / kGroup;
      if (rg < nrg && !(dense[l] && (tid >> 7)))
        kp[l][tid >> 7][tid & 127] = c.s[l].params[(int64_t(rg) * H + h) * kAttnD + (tid & 127)];
    }
  }

  // issue every item's code word (and V parameter, and compact position) up front
  uint32_t cw[NL][4], vp[NL][4];
  int32_t pos[NL][4];
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t j = lo[l] + ts + 16 * i;               // row of the stream
      const bool ok = l < nl && j < hi[l];
      cw[l][i] = 0;
      vp[l][i] = 0;
      pos[l][i] = -1;
      if (ok) {
        cw[l][i] = *reinterpret_cast<const uint32_t*>(c.s[l].codes + (int64_t(j) * H + h) * (kAttnD / 2) + oc * 4);
        if (KIND == FLK_KIND_V) vp[l][i] = c.s[l].params[(int64_t(j) * H + h) * 2 + (oc >> 3)];
        pos[l][i] = dense[l] ? j - t0 : c.s[l].rows[j] - t0;
      }
    }
  if (KIND == FLK_KIND_K) __syncthreads();                // staged parameter rows visible

  auto params_of = [&](int l, int32_t j, uint32_t p[8]) {
    if (KIND == FLK_KIND_K) {
      const int r = j / kGroup - lo[l] / kGroup;
      const uint4 a = *reinterpret_cast<const uint4*>(&kp[l][r][oc * 8]);
      const uint4 b = *reinterpret_cast<const uint4*>(&kp[l][r][oc * 8 + 4]);
      p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w; p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = 0;
    }
  };

  // leading dense loops in registers; tokens past T stay zero
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (l >= dp) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (pos[l][i] < 0) continue;
      uint32_t p[8];
      params_of(l, lo[l] + ts + 16 * i, p);
      if (KIND == FLK_KIND_V) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = vp[l][i];
      }
      float d[8];
      decode_item(cw[l][i], p, d);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = l == 0 ? d[e] : round_bf16(acc[i][e] + d[e]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) store_bf16x8(&s[ts + 16 * i][oc * 8], acc[i]);
  __syncthreads();

  // every later loop: read-modify-write of the rows it lists
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (l < dp || l >= nl) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t pl = uint32_t(pos[l][i]);
      if (pl >= uint32_t(kGroup)) continue;               // no row, or a map entry outside the tile
      uint32_t p[8];
      params_of(l, lo[l] + ts + 16 * i, p);
      if (KIND == FLK_KIND_V) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = vp[l][i];
      }
      float d[8], v[8];
      decode_item(cw[l][i], p, d);
      load_bf16x8(&s[pl][oc * 8], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = round_bf16(v[e] + d[e]);
      store_bf16x8(&s[pl][oc * 8], v);
    }
    __syncthreads();
  }
}

template <int NL>
__global__ __launch_bounds__(kAThreads) void attn_tile_kernel(ChainArgs kc, ChainArgs vc, int32_t T, int32_t H,
                                                              int32_t G, const uint16_t* __restrict__ q,
                                                              float scale, int32_t tps,
                                                              float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  __shared__ __attribute__((aligned(16))) uint16_t s_kv[2][kGroup][kLdsRow];
  __shared__ __attribute__((aligned(16))) uint32_t s_kp[NL][2][kAttnD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 15;                                // query head of this lane (MFMA column)
  const int kb = lane >> 4;                               // k-block / row block of this lane
  const int32_t split = blockIdx.x;
  const int32_t h = blockIdx.y;
  const int32_t Hq = H * G;
  const int32_t tiles = (T + kGroup - 1) / kGroup;
  const int32_t tile0 = split * tps;
  const int32_t tile1 = min(tiles, tile0 + tps);

  // Q^T as the B operand of S^T = K_hat Q^T: lane holds Q[n][32*ks + 8*kb + j], zero past G
  bf16x8_t qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < G) w = *reinterpret_cast<const uint4*>(q + int64_t(h * G + n) * kAttnD + 32 * ks + 8 * kb);
    qb[ks] = __builtin_bit_cast(bf16x8_t, w);
  }

  float m_run = -__builtin_inff(), l_run = 0.0f;
  float4_t o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int32_t tile = tile0; tile < tile1; ++tile) {
    decode_tile<FLK_KIND_K, NL>(kc, tile, T, H, h, s_kv[0], s_kp);
    decode_tile<FLK_KIND_V, NL>(vc, tile, T, H, h, s_kv[1], s_kp);

    // scores of this wave's 16 tokens: S^T[token][head], lane holds tokens 4*kb + i of head n
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(&s_kv[0][16 * wave + n][32 * ks + 8 * kb]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qb[ks], sacc, 0, 0, 0);
    }
    float sc[4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t t = tile * kGroup + 16 * wave + 4 * kb + i;
      sc[i] = t < T ? sacc[i] * scale : -__builtin_inff();
      mx = fmaxf(mx, sc[i]);
    }
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

    // O^T[ch][head] += V_hat^T[ch][token] P^T[token][head]; lane: channel 16*mt + n, tokens 4*kb + j
    short4_t pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) pb[j] = short(__builtin_bit_cast(uint16_t, (__bf16)p[j]));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      short4_t a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = short(s_kv[1][16 * wave + 4 * kb + j][16 * mt + n]);
      o[mt] = o[mt] * corr;
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[mt], 0, 0, 0);
    }
    __syncthreads();                                      // LDS tiles are rewritten next
  }

  // merge the 4 waves: (m, l) per head and O^T per (head, channel) through LDS
  float* s_m = reinterpret_cast<float*>(&s_kv[0][0][0]);  // [4][16]
  float* s_l = s_m + 4 * kMaxG;                           // [4][16]
  float* s_o = s_l + 4 * kMaxG;                           // [4][16][128]
  if (kb == 0) {
    s_m[wave * kMaxG + n] = m_run;
    s_l[wave * kMaxG + n] = l_run;
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[(wave * kMaxG + n) * kAttnD + 16 * mt + 4 * kb + i] = o[mt][i];
  __syncthreads();
  for (int idx = tid; idx < G * kAttnD; idx += kAThreads) {
    const int g = idx / kAttnD, ch = idx % kAttnD;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w * kMaxG + g]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_m[w * kMaxG + g];
      const float f = mw == -__builtin_inff() ? 0.0f : __expf(mw - M);
      L += s_l[w * kMaxG + g] * f;
      O += s_o[(w * kMaxG + g) * kAttnD + ch] * f;
    }
    const int64_t qi = int64_t(split) * Hq + h * G + g;
    if (ch == 0) { ws_ml[2 * qi] = M; ws_ml[2 * qi + 1] = L; }
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
                                                                            uint16_t* __restrict__ out) {
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
  }
}

hipError_t launch_decode_attn(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, float scale, void* out,
                              void* ws, hipStream_t stream) {
  (void)D;
  const int32_t tps = tiles_per_split(T, H);
  const int32_t splits = n_splits(T, H);
  const int32_t G = Hq / H;
  float* ws_ml = static_cast<float*>(ws);
  float* ws_o = ws_ml + size_t(splits) * Hq * 2;
  const int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  const dim3 grid(static_cast<unsigned>(splits), static_cast<unsigned>(H));
  const uint16_t* qp = static_cast<const uint16_t*>(q);
#define FLK_A(NLV)                                                                                      \
  case NLV:                                                                                             \
    hipLaunchKernelGGL((attn_tile_kernel<NLV>), grid, dim3(kAThreads), 0, stream, kc, vc, T, H, G, qp, \
                       scale, tps, ws_ml, ws_o);                                                        \
    break;
  switch (nl) {
    FLK_A(1) FLK_A(2) FLK_A(3) FLK_A(4) FLK_A(5) FLK_A(6) FLK_A(7) FLK_A(8)
    default: return hipErrorInvalidValue;
  }
#undef FLK_A
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(Hq), dim3(kAttnD * kCombGroups), 0, stream, splits, Hq, ws_ml,
                     ws_o, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace flk
