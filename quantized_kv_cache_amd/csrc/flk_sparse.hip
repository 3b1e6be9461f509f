// flk_sparse.hip -- sparse decode attention over packed chains (FlashLoop RFC, vllm-rlt #156,
// section 3.2 "Sparse decode attention").
//
// Reference loop: the packed-chain attention kernel runs full attention and also writes every
// scaled score; topk_kernel selects, per query head, the k highest scores (equal scores by the
// lower position) with a three-pass radix select and a position-ordered compaction; the gather
// kernel then sums the selected keys' reference probabilities (m) and weighted values (C_ref).
// Later loop: the gather kernel reads the selected keys alone through the chain at that loop's
// depth -- K for the scores, V for the weighted sum, online softmax in binary32 -- and the
// combine applies O = O_ref - C_ref + m * (p_local . V_S).
//
// A selected position's compact row in a compact loop comes from a position -> row map that
// chain_map_kernel writes per call (one wave per 64-position tile), so a gather reads one map
// entry per loop instead of searching.
#include "flk_device.h"
#include "flk_internal.h"

namespace flk {

constexpr int kSD = 128;                     // head dimension
constexpr int kSThreads = 256;
constexpr int kSWaves = kSThreads / 64;
constexpr int kKeysPerWave = 32;             // two 16-key slices per wave
constexpr int kKeysPerBlock = kKeysPerWave * kSWaves;
constexpr int kTopThreads = 1024;

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------------------
// Top-k per query head.  Scores map to unsigned keys whose order is the scores' order; a
// radix select over three digits (bits 31..21, 20..10, 9..0) finds the k-th largest key tau
// and how many keys equal to tau belong to S (the lowest positions among them); a final pass
// writes S in position order (a block-wide scan of each thread's counts over its contiguous
// chunk).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan of one value per thread across the block (Hillis-Steele in LDS).
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTopThreads; off <<= 1) {
    const uint32_t add = tid >= off ? buf[tid - off] : 0u;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const uint32_t r = buf[tid];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTopThreads) void topk_kernel(const float* __restrict__ scores, int32_t T, int32_t k,
                                                           int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t buf[kTopThreads];
  __shared__ uint32_t s_digit, s_above;
  const int tid = threadIdx.x;
  const int32_t qh = blockIdx.x;
  const float* sc = scores + int64_t(qh) * T;
  uint32_t prefix = 0, pmask = 0, need = uint32_t(k);
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const uint32_t nb = pass == 2 ? 1024u : 2048u;
    for (int b = tid; b < 2048; b += kTopThreads) hist[b] = 0;
    __syncthreads();
    for (int32_t t = tid; t < T; t += kTopThreads) {
      const uint32_t key = order_key(sc[t]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // counts from the top digit down: thread t owns digits nb-1-2t and nb-2-2t
    const int32_t d0 = int32_t(nb) - 1 - 2 * tid, d1 = d0 - 1;
    const uint32_t c0 = d0 >= 0 ? hist[d0] : 0u, c1 = d1 >= 0 ? hist[d1] : 0u;
    const uint32_t incl = block_scan_incl(c0 + c1, buf);
    const uint32_t before0 = incl - c0 - c1, before1 = before0 + c0;
    if (d0 >= 0 && before0 < need && need <= before0 + c0) { s_digit = uint32_t(d0); s_above = before0; }
    if (d1 >= 0 && before1 < need && need <= before1 + c1) { s_digit = uint32_t(d1); s_above = before1; }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= (nb - 1) << shift;
    need -= s_above;
    __syncthreads();
  }
  // prefix is tau; `need` keys equal to tau are selected, the lowest positions first
  const int32_t chunk = (T + kTopThreads - 1) / kTopThreads;
  const int32_t c_lo = min(T, tid * chunk), c_hi = min(T, c_lo + chunk);
  uint32_t gt = 0, eq = 0;
  for (int32_t t = c_lo; t < c_hi; ++t) {
    const uint32_t key = order_key(sc[t]);
    gt += key > prefix;
    eq += key == prefix;
  }
  const uint32_t g0 = block_scan_incl(gt, buf) - gt;
  const uint32_t e0 = block_scan_incl(eq, buf) - eq;
  uint32_t out = g0 + min(e0, need), e = e0;
  int32_t* dst = sel + int64_t(qh) * k;
  for (int32_t t = c_lo; t < c_hi; ++t) {
    const uint32_t key = order_key(sc[t]);
    bool take = key > prefix;
    if (key == prefix) take = e++ < need;
    if (take && out < uint32_t(k)) dst[out++] = t;
  }
}

// ---------------------------------------------------------------------------------------
// Position -> compact row maps of a chain's compact loops.
// ---------------------------------------------------------------------------------------
struct MapJob {
  const int32_t* rows;
  const int32_t* tile_start;
  int32_t* map;                 // [T] compact row of each position, -1 where the loop is absent
  int32_t n;
};
constexpr int kMaxMapJobs = 2 * FLK_MAX_LOOPS;
struct MapJobs {
  MapJob j[kMaxMapJobs];
  int32_t n_jobs, T;
};

__global__ __launch_bounds__(kSThreads) void chain_map_kernel(MapJobs jobs) {
  __shared__ int32_t slot[kSWaves][kGroup];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const MapJob& m = jobs.j[blockIdx.y];
  const int32_t T = jobs.T;
  const int32_t ntiles = (T + kGroup - 1) / kGroup;
  const int32_t tile = int32_t(blockIdx.x) * kSWaves + wave;
  if (tile >= ntiles) return;                               // wave-uniform; no block barrier below
  const int32_t lo = min(max(m.tile_start[tile], 0), m.n);
  const int32_t hi = min(max(m.tile_start[tile + 1], lo), min(m.n, lo + kGroup));
  slot[wave][lane] = -1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int32_t j = lo + lane;
  if (j < hi) {
    const uint32_t o = uint32_t(m.rows[j] - tile * kGroup);
    if (o < uint32_t(kGroup)) slot[wave][o] = j;           // a malformed entry outside the tile is dropped
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int32_t p = tile * kGroup + lane;
  if (p < T) m.map[p] = slot[wave][lane];
}

// ---------------------------------------------------------------------------------------
// Gather: the selected keys of one query head, read through the chain at the call's depth.
// A block covers 128 keys of one query head (4 waves x two 16-key slices).  Lane (n, kb) =
// (lane & 15, lane >> 4) holds key n of the slice, channel octets kb, kb + 4, kb + 8, kb + 12
// (32 channels); a key's score is summed over its 4 kb lanes, a slice's softmax over the 16 n
// lanes, and each lane accumulates its own 32 output channels.
// ---------------------------------------------------------------------------------------
struct GatherArgs {
  ChainArgs kc, vc;
  const int32_t* kmap[FLK_MAX_LOOPS];   // position -> compact row per compact loop, else nullptr
  const int32_t* vmap[FLK_MAX_LOOPS];
  const uint16_t* q;                    // loop: [Hq][128]
  const int32_t* sel;                   // [Hq][k]
  const float* scores;                  // reference: [Hq][T]
  const float* ml;                      // reference: [Hq][2] softmax max and denominator
  float* part;                          // per (head, block) partials
  int32_t T, H, G, k, nblk;
  float scale;
};

// 8 channels (octet oc) of key position p of KV head h at the chain's depth, as binary32 values
// that are exactly the BF16 reconstruction.
template <int KIND, int NL>
__device__ __forceinline__ void gather_octet(const ChainArgs& c, const int32_t* const* maps, int32_t p, int32_t H,
                                             int32_t h, int oc, float acc[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (l >= c.n_loops) continue;
    const StreamArgs& st = c.s[l];
    const int32_t j = st.rows == nullptr ? p : maps[l][p];
    if (j < 0) continue;                                     // absent: inherits
    const uint32_t item = uint32_t(j) * uint32_t(H) + uint32_t(h);
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(st.codes + (item * (kSD / 2) + uint32_t(oc) * 4u));
    uint32_t pw[8];
    if (KIND == FLK_KIND_K) {
      const uint32_t row = c.ktile ? uint32_t(p) / kGroup : uint32_t(j) / kGroup;
      const uint4* pp = reinterpret_cast<const uint4*>(st.params + (row * uint32_t(H) + uint32_t(h)) * kSD + uint32_t(oc) * 8u);
      const uint4 a = pp[0], b = pp[1];
      pw[0] = a.x; pw[1] = a.y; pw[2] = a.z; pw[3] = a.w; pw[4] = b.x; pw[5] = b.y; pw[6] = b.z; pw[7] = b.w;
    } else {
      const uint32_t w = st.params[item * 2u + uint32_t(oc >> 3)];
#pragma unroll
      for (int e = 0; e < 8; ++e) pw[e] = w;
    }
    float cv[8], d[8];
    codes8_to_f32(cw, cv);
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = decode(cv[e], f16_bits_to_f32(pw[e] & 0xFFFFu), f16_bits_to_f32(pw[e] >> 16));
    round_bf16x8_inplace(d);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = l == 0 ? d[e] : round_bf16(acc[e] + d[e]);
  }
}

__device__ __forceinline__ float sum16(float v) {          // over lane bits 0..3
  v += dpp_xor1(v);
  v += dpp_xor2(v);
  v += dpp_half_mirror(v);
  v += dpp_ror8(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  v = fmaxf(v, dpp_half_mirror(v));
  v = fmaxf(v, dpp_ror8(v));
  return v;
}

// MODE 0 (reference statistics): partial (mass, c[128]) of p_t = exp(s_t - M) / L over the keys.
// MODE 1 (later loop): partial (m, l, o[128]) of the online softmax over the keys.
template <int NL, int MODE>
__global__ __launch_bounds__(kSThreads) void sparse_gather_kernel(GatherArgs g) {
  __shared__ float s_m[kSWaves], s_l[kSWaves];
  __shared__ float s_o[kSWaves][kSD];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int32_t qh = blockIdx.y, h = qh / g.G;
  const int32_t key0 = int32_t(blockIdx.x) * kKeysPerBlock + wave * kKeysPerWave;
  const int32_t* sel = g.sel + int64_t(qh) * g.k;

  float qv[32];
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(g.q + int64_t(qh) * kSD + (4 * i + kb) * 8);
      qv[8 * i + 0] = bf16_lo(w.x); qv[8 * i + 1] = bf16_hi(w.x);
      qv[8 * i + 2] = bf16_lo(w.y); qv[8 * i + 3] = bf16_hi(w.y);
      qv[8 * i + 4] = bf16_lo(w.z); qv[8 * i + 5] = bf16_hi(w.z);
      qv[8 * i + 6] = bf16_lo(w.w); qv[8 * i + 7] = bf16_hi(w.w);
    }
  }
  float M = 0.0f, Linv = 0.0f;
  if (MODE == 0) {
    M = g.ml[2 * qh];
    Linv = 1.0f / g.ml[2 * qh + 1];
  }
  float m_run = MODE == 1 ? -__builtin_inff() : 0.0f;       // mode 0: the mass
  float l_run = 0.0f;
  float o[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) o[c] = 0.0f;

  for (int sl = 0; sl < kKeysPerWave / 16; ++sl) {
    const int32_t r = key0 + 16 * sl + n;
    int32_t p = -1;
    if (r < g.k) {
      p = sel[r];
      if (uint32_t(p) >= uint32_t(g.T)) p = -1;             // out of range: skipped
    }
    if (MODE == 1) {
      float s = 0.0f;
      if (p >= 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float kv[8];
          gather_octet<FLK_KIND_K, NL>(g.kc, g.kmap, p, g.H, h, 4 * i + kb, kv);
#pragma unroll
          for (int e = 0; e < 8; ++e) s = __builtin_fmaf(qv[8 * i + e], kv[e], s);
        }
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      s = p >= 0 ? s * g.scale : -__builtin_inff();
      const float m_new = fmaxf(m_run, max16(s));
      const float corr = m_run == -__builtin_inff() ? 0.0f : __expf(m_run - m_new);
      const float pn = p >= 0 ? __expf(s - m_new) : 0.0f;
      l_run = l_run * corr + sum16(pn);
      m_run = m_new;
#pragma unroll
      for (int c = 0; c < 32; ++c) o[c] *= corr;
      if (p >= 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float vv[8];
          gather_octet<FLK_KIND_V, NL>(g.vc, g.vmap, p, g.H, h, 4 * i + kb, vv);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[8 * i + e] = __builtin_fmaf(pn, vv[e], o[8 * i + e]);
        }
      }
    } else {
      const float w = p >= 0 ? __expf(g.scores[int64_t(qh) * g.T + p] - M) * Linv : 0.0f;
      m_run += sum16(w);
      if (p >= 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float vv[8];
          gather_octet<FLK_KIND_V, NL>(g.vc, g.vmap, p, g.H, h, 4 * i + kb, vv);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[8 * i + e] = __builtin_fmaf(w, vv[e], o[8 * i + e]);
        }
      }
    }
  }
  // this wave's output channels: sum over the 16 keys of the slice lanes
#pragma unroll
  for (int c = 0; c < 32; ++c) o[c] = sum16(o[c]);
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][(4 * i + kb) * 8 + e] = o[8 * i + e];
    if (kb == 0) {
      s_m[wave] = m_run;
      s_l[wave] = l_run;
    }
  }
  __syncthreads();
  // merge the 4 waves into the block's partial
  float* part = g.part + (int64_t(qh) * g.nblk + blockIdx.x) * (2 + kSD);
  const int c = threadIdx.x;
  if (MODE == 1) {
    float Mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) Mx = fmaxf(Mx, s_m[w]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) {
      const float f = s_m[w] == -__builtin_inff() ? 0.0f : __expf(s_m[w] - Mx);
      L += s_l[w] * f;
      if (c < kSD) O += s_o[w][c] * f;
    }
    if (c < kSD) part[2 + c] = O;
    if (c == 0) { part[0] = Mx; part[1] = L; }
  } else {
    float mass = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) {
      mass += s_m[w];
      if (c < kSD) O += s_o[w][c];
    }
    if (c < kSD) part[2 + c] = O;
    if (c == 0) { part[0] = mass; part[1] = 0.0f; }
  }
}

// Per query head (block), thread c = channel: merge the blocks' partials.
// MODE 0: mass[qh] = sum of masses, c_ref[qh][c] = sum.  MODE 1: out = O_ref - C_ref + m * o / l.
template <int MODE>
__global__ __launch_bounds__(kSD) void sparse_combine_kernel(const float* __restrict__ part, int32_t nblk,
                                                             float* __restrict__ mass_out, float* __restrict__ c_out,
                                                             const float* __restrict__ mass,
                                                             const float* __restrict__ o_ref,
                                                             const float* __restrict__ c_ref,
                                                             uint16_t* __restrict__ out) {
  const int32_t qh = blockIdx.x;
  const int c = threadIdx.x;
  const float* pp = part + int64_t(qh) * nblk * (2 + kSD);
  if (MODE == 0) {
    float m = 0.0f, O = 0.0f;
    for (int32_t b = 0; b < nblk; ++b) {
      m += pp[b * (2 + kSD)];
      O += pp[b * (2 + kSD) + 2 + c];
    }
    c_out[int64_t(qh) * kSD + c] = O;
    if (c == 0) mass_out[qh] = m;
  } else {
    float Mx = -__builtin_inff();
    for (int32_t b = 0; b < nblk; ++b) Mx = fmaxf(Mx, pp[b * (2 + kSD)]);
    float L = 0.0f, O = 0.0f;
    for (int32_t b = 0; b < nblk; ++b) {
      const float mb = pp[b * (2 + kSD)];
      const float f = mb == -__builtin_inff() ? 0.0f : __expf(mb - Mx);
      L += pp[b * (2 + kSD) + 1] * f;
      O += pp[b * (2 + kSD) + 2 + c] * f;
    }
    const int64_t i = int64_t(qh) * kSD + c;
    const float c_new = L > 0.0f ? mass[qh] * (O / L) : 0.0f;
    out[i] = __builtin_bit_cast(uint16_t, (__bf16)(o_ref[i] - c_ref[i] + c_new));
  }
}

// ---------------------------------------------------------------------------------------
// Host side.  Workspace: [maps K][maps V][partials] for every call, and for the reference
// [attention partials][scores][ml] after them.
// ---------------------------------------------------------------------------------------
static int32_t gather_blocks(int32_t k) { return (k + kKeysPerBlock - 1) / kKeysPerBlock; }

struct SparseLayout {
  size_t kmaps, vmaps, part, attn, scores, ml, total;
};
static SparseLayout sparse_layout(int32_t T, int32_t H, int32_t Hq, int32_t k, int32_t n_loops) {
  SparseLayout L{};
  size_t off = 0;
  const size_t map_bytes = align256(size_t(T) * sizeof(int32_t)) * size_t(n_loops);
  L.kmaps = off; off += map_bytes;
  L.vmaps = off; off += map_bytes;
  L.part = off; off += align256(size_t(Hq) * gather_blocks(k) * (2 + kSD) * sizeof(float));
  L.attn = off; off += align256(attn_workspace_bytes(T, H, Hq));
  L.scores = off; off += align256(size_t(Hq) * size_t(T) * sizeof(float));
  L.ml = off; off += align256(size_t(Hq) * 2 * sizeof(float));
  L.total = off;
  return L;
}

size_t sparse_workspace_bytes(int32_t T, int32_t H, int32_t Hq, int32_t k, int32_t n_loops) {
  return sparse_layout(T, H, Hq, k, n_loops).total;
}

static hipError_t build_maps(const ChainArgs& c, int32_t T, int32_t* base, const int32_t** maps, hipStream_t stream) {
  MapJobs jobs{};
  jobs.T = T;
  const size_t stride = align256(size_t(T) * sizeof(int32_t)) / sizeof(int32_t);
  for (int l = 0; l < FLK_MAX_LOOPS; ++l) maps[l] = nullptr;
  for (int l = 0; l < c.n_loops; ++l) {
    if (c.s[l].rows == nullptr) continue;
    int32_t* m = base + size_t(l) * stride;
    jobs.j[jobs.n_jobs++] = MapJob{c.s[l].rows, c.s[l].tile_start, m, c.s[l].n};
    maps[l] = m;
  }
  if (jobs.n_jobs == 0) return hipSuccess;
  const int32_t ntiles = (T + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(chain_map_kernel, dim3(unsigned((ntiles + kSWaves - 1) / kSWaves), unsigned(jobs.n_jobs)),
                     dim3(kSThreads), 0, stream, jobs);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gather(const GatherArgs& g, int nl, hipStream_t stream) {
  const dim3 grid(unsigned(g.nblk), unsigned(g.H * g.G));
#define FLK_G(NLV)                                                                                        \
  case NLV:                                                                                               \
    hipLaunchKernelGGL((sparse_gather_kernel<NLV, MODE>), grid, dim3(kSThreads), 0, stream, g);         \
    break;
  switch (nl) {
    FLK_G(1) FLK_G(2) FLK_G(3) FLK_G(4) FLK_G(5) FLK_G(6) FLK_G(7) FLK_G(8)
    default: return hipErrorInvalidValue;
  }
#undef FLK_G
  return hipGetLastError();
}

hipError_t launch_sparse_reference(int32_t T, int32_t H, int32_t Hq, int32_t k, const void* q, const ChainArgs& kc,
                                   const ChainArgs& vc, float scale, void* out, int32_t* sel, float* mass,
                                   float* o_ref, float* c_ref, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  const SparseLayout L = sparse_layout(T, H, Hq, k, nl);
  if (ws == nullptr || ws_bytes < L.total || k < 1 || k > T) return hipErrorInvalidValue;
  char* w = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(w + L.scores);
  float* ml = reinterpret_cast<float*>(w + L.ml);
  hipError_t e = launch_attn_reference(T, H, Hq, q, kc, vc, scale, out, o_ref, ml, scores, w + L.attn,
                                       attn_workspace_bytes(T, H, Hq), stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3(unsigned(Hq)), dim3(kTopThreads), 0, stream, scores, T, k, sel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  GatherArgs g{};
  g.kc = kc;
  g.vc = vc;
  if ((e = build_maps(vc, T, reinterpret_cast<int32_t*>(w + L.vmaps), g.vmap, stream)) != hipSuccess) return e;
  g.sel = sel;
  g.scores = scores;
  g.ml = ml;
  g.part = reinterpret_cast<float*>(w + L.part);
  g.T = T;
  g.H = H;
  g.G = Hq / H;
  g.k = k;
  g.nblk = gather_blocks(k);
  g.scale = scale;
  if ((e = launch_gather<0>(g, vc.n_loops, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_combine_kernel<0>), dim3(unsigned(Hq)), dim3(kSD), 0, stream, g.part, g.nblk, mass,
                     c_ref, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_sparse_loop(int32_t T, int32_t H, int32_t Hq, int32_t k, const void* q, const ChainArgs& kc,
                              const ChainArgs& vc, float scale, const int32_t* sel, const float* mass,
                              const float* o_ref, const float* c_ref, void* out, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  const int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  const SparseLayout L = sparse_layout(T, H, Hq, k, nl);
  if (ws == nullptr || ws_bytes < L.part + align256(size_t(Hq) * gather_blocks(k) * (2 + kSD) * sizeof(float)) ||
      k < 1 || k > T)
    return hipErrorInvalidValue;
  char* w = static_cast<char*>(ws);
  GatherArgs g{};
  g.kc = kc;
  g.vc = vc;
  hipError_t e = build_maps(kc, T, reinterpret_cast<int32_t*>(w + L.kmaps), g.kmap, stream);
  if (e != hipSuccess) return e;
  if ((e = build_maps(vc, T, reinterpret_cast<int32_t*>(w + L.vmaps), g.vmap, stream)) != hipSuccess) return e;
  g.q = static_cast<const uint16_t*>(q);
  g.sel = sel;
  g.part = reinterpret_cast<float*>(w + L.part);
  g.T = T;
  g.H = H;
  g.G = Hq / H;
  g.k = k;
  g.nblk = gather_blocks(k);
  g.scale = scale;
  if ((e = launch_gather<1>(g, nl, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_combine_kernel<1>), dim3(unsigned(Hq)), dim3(kSD), 0, stream, g.part, g.nblk, nullptr,
                     nullptr, mass, o_ref, c_ref, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace flk
