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
#include "flk_blockscan.h"
#include "flk_device.h"
#include "flk_fp4_device.h"
#include "flk_internal.h"
#include "flk_readers.h"

namespace flk {

constexpr int kSD = 128;                     // head dimension
constexpr int kSThreads = 256;
constexpr int kSWaves = kSThreads / 64;
#ifndef FLK_SPARSE_KPW
#define FLK_SPARSE_KPW 16
#endif
constexpr int kKeysPerWave = FLK_SPARSE_KPW;  // one 16-key slice per wave: more, shorter waves
constexpr int kKeysPerBlock = kKeysPerWave * kSWaves;
constexpr int kTopThreads = 1024;

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// Floats between two query heads' rows of reference scores (16-byte aligned rows).
__host__ __device__ __forceinline__ int64_t score_stride(int32_t T) { return (int64_t(T) + 3) & ~int64_t(3); }

// ---------------------------------------------------------------------------------------
// Top-k per query head.  Scores map to unsigned keys whose order is the scores' order; a
// radix select over three digits (bits 31..21, 20..10, 9..0) finds the k-th largest key tau
// and how many keys equal to tau belong to S (the lowest positions among them); a final pass
// writes S in position order, each wave over a contiguous segment, counting with ballots 64
// coalesced values at a time.  Every pass keeps kTopBatch loads in flight per thread: with one
// block per head nothing else hides the memory latency.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopWaves = kTopThreads / 64;
constexpr int kTopBatch = 8;                 // 16-byte score loads in flight per thread

// Four consecutive scores t..t+3 of a row as keys (t a multiple of 4); positions at or past T
// give key 0, below every real score's key.
__device__ __forceinline__ void keys4(const float* __restrict__ sc, int32_t t, int32_t T, uint32_t k[4]) {
  if (t + 3 < T) {
    const float4 v = *reinterpret_cast<const float4*>(sc + t);
    k[0] = order_key(v.x); k[1] = order_key(v.y); k[2] = order_key(v.z); k[3] = order_key(v.w);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) k[e] = t + e < T ? order_key(sc[t + e]) : 0u;
  }
}

// Sum over the lanes below this one of a per-lane count 0..7, from three ballots of its bits.
__device__ __forceinline__ uint32_t lanes_below_sum(uint32_t c, uint64_t below) {
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < 3; ++b) r += uint32_t(__builtin_popcountll(__ballot((c >> b) & 1u) & below)) << b;
  return r;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t c) {
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < 3; ++b) r += uint32_t(__builtin_popcountll(__ballot((c >> b) & 1u))) << b;
  return r;
}

// Rows of scores are ceil(T/4)*4 floats apart (16-byte aligned) and read 4 at a time.
__global__ __launch_bounds__(kTopThreads) void topk_kernel(const float* __restrict__ scores, int32_t T, int32_t k,
                                                           int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_cnt[kTopWaves][2];
  __shared__ uint32_t s_digit, s_above;
  __shared__ int32_t s_tmp[kTopWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  const int32_t qh = blockIdx.x;
  const float* sc = scores + int64_t(qh) * score_stride(T);
  uint32_t prefix = 0, pmask = 0, need = uint32_t(k);
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const uint32_t nb = pass == 2 ? 1024u : 2048u;
    for (int b = tid; b < 2048; b += kTopThreads) hist[b] = 0;
    __syncthreads();
    for (int32_t t0 = 0; t0 < T; t0 += 4 * kTopThreads * kTopBatch) {
      uint32_t key[kTopBatch][4];
#pragma unroll
      for (int i = 0; i < kTopBatch; ++i) keys4(sc, t0 + 4 * (i * kTopThreads + tid), T, key[i]);
#pragma unroll
      for (int i = 0; i < kTopBatch; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int32_t t = t0 + 4 * (i * kTopThreads + tid) + e;
          if (t < T && (key[i][e] & pmask) == prefix) atomicAdd(&hist[(key[i][e] >> shift) & (nb - 1)], 1u);
        }
    }
    __syncthreads();
    uint32_t digit, above;                                   // from the top digit down to the k-th key
    block_find_digit<kTopThreads>(hist, nb, need, s_tmp, digit, above, &s_digit, &s_above);
    prefix |= digit << shift;
    pmask |= (nb - 1) << shift;
    need -= above;
    __syncthreads();
  }
  // prefix is tau; `need` keys equal to tau are selected, the lowest positions first.  Wave w
  // owns the contiguous segment [w*seg, (w+1)*seg) of positions, 256 of them per step (lane l
  // holds positions 4l..4l+3 of the step).
  const int32_t seg = ((T + kTopWaves - 1) / kTopWaves + 255) & ~255;
  const int32_t lo = min(T, wave * seg), hi = min(T, lo + seg);
  uint32_t gt = 0, eq = 0;
  for (int32_t t0 = lo; t0 < hi; t0 += 256 * kTopBatch) {
    uint32_t key[kTopBatch][4];
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) keys4(sc, t0 + 256 * i + 4 * lane, hi, key[i]);
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) {
      uint32_t g = 0, q = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = t0 + 256 * i + 4 * lane + e < hi;
        g += in && key[i][e] > prefix;
        q += in && key[i][e] == prefix;
      }
      gt += wave_sum(g);
      eq += wave_sum(q);
    }
  }
  if (lane == 0) { s_cnt[wave][0] = gt; s_cnt[wave][1] = eq; }
  __syncthreads();
  uint32_t g0 = 0, e0 = 0;
  for (int w = 0; w < wave; ++w) { g0 += s_cnt[w][0]; e0 += s_cnt[w][1]; }
  int32_t* dst = sel + int64_t(qh) * k;
  uint32_t out = g0 + min(e0, need), e_seen = e0;
  for (int32_t t0 = lo; t0 < hi; t0 += 256 * kTopBatch) {
    uint32_t key[kTopBatch][4];
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) keys4(sc, t0 + 256 * i + 4 * lane, hi, key[i]);
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) {
      const int32_t tb = t0 + 256 * i + 4 * lane;
      bool is_eq[4];
      uint32_t q = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        is_eq[e] = tb + e < hi && key[i][e] == prefix;
        q += is_eq[e];
      }
      uint32_t eq_rank = e_seen + lanes_below_sum(q, below);   // equal keys before this lane's
      bool take[4];
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        take[e] = (tb + e < hi && key[i][e] > prefix) || (is_eq[e] && eq_rank < need);
        eq_rank += is_eq[e];
        c += take[e];
      }
      uint32_t slot = out + lanes_below_sum(c, below);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (take[e]) {
          if (slot < uint32_t(k)) dst[slot] = tb + e;
          ++slot;
        }
      out += wave_sum(c);
      e_seen += wave_sum(q);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Top-k split over segments, for long rows: one block of 1024 threads per head keeps a single
// CU busy with three passes of LDS atomics over T keys, so past kSplitMinT each head's row
// is cut into B segments of S keys (S a multiple of 4).  Per radix pass, topk_seg_hist_kernel
// builds each segment's digit histogram (of the keys that match the head's prefix so far) and
// topk_seg_digit_kernel sums a head's segment histograms and advances its state {prefix,
// mask, need}; then topk_seg_count_kernel counts each segment's keys above and equal to tau,
// and topk_seg_write_kernel writes the segment's selected positions at offsets taken from the
// earlier segments' counts.  The selection is exactly the one-block kernel's.
// ---------------------------------------------------------------------------------------
constexpr int32_t kSplitMinT = 16384;
constexpr int32_t kSegKeys = 8192;            // target keys per segment
constexpr int kSegThreads = 256;
constexpr int kSegWaves = kSegThreads / 64;

struct SplitTopk {
  int32_t B, S;                               // segments per head, keys per segment
};
__host__ __device__ inline SplitTopk split_topk(int32_t T) {
  SplitTopk t;
  t.B = (T + kSegKeys - 1) / kSegKeys;
  if (t.B > 64) t.B = 64;
  t.S = (((T + t.B - 1) / t.B) + 3) & ~3;
  return t;
}

__device__ __forceinline__ void pass_digits(int pass, int& shift, uint32_t& nb) {
  shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
  nb = pass == 2 ? 1024u : 2048u;
}

__global__ __launch_bounds__(kSegThreads) void topk_seg_hist_kernel(const float* __restrict__ scores, int32_t T,
                                                                     int32_t B, int32_t S, int pass,
                                                                     const uint32_t* __restrict__ state,
                                                                     uint32_t* __restrict__ ghist) {
  __shared__ uint32_t hist[2048];
  const int tid = threadIdx.x;
  const int32_t b = blockIdx.x, qh = blockIdx.y;
  const float* sc = scores + int64_t(qh) * score_stride(T);
  int shift;
  uint32_t nb;
  pass_digits(pass, shift, nb);
  const uint32_t prefix = pass ? state[4 * qh] : 0u, pmask = pass ? state[4 * qh + 1] : 0u;
  for (int d = tid; d < 2048; d += kSegThreads) hist[d] = 0;
  __syncthreads();
  const int32_t lo = b * S, hi = min(T, lo + S);
  for (int32_t t0 = lo; t0 < hi; t0 += 4 * kSegThreads * kTopBatch) {
    uint32_t key[kTopBatch][4];
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) keys4(sc, t0 + 4 * (i * kSegThreads + tid), hi, key[i]);
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int32_t t = t0 + 4 * (i * kSegThreads + tid) + e;
        if (t < hi && (key[i][e] & pmask) == prefix) atomicAdd(&hist[(key[i][e] >> shift) & (nb - 1)], 1u);
      }
  }
  __syncthreads();
  uint32_t* dst = ghist + (int64_t(qh) * B + b) * 2048;
  for (int d = tid; d < int(nb); d += kSegThreads) dst[d] = hist[d];
}

__global__ __launch_bounds__(kTopThreads) void topk_seg_digit_kernel(int32_t B, int32_t k, int pass,
                                                                      const uint32_t* __restrict__ ghist,
                                                                      uint32_t* __restrict__ state) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_digit, s_above;
  __shared__ int32_t s_tmp[kTopWaves];
  const int tid = threadIdx.x;
  const int32_t qh = blockIdx.x;
  int shift;
  uint32_t nb;
  pass_digits(pass, shift, nb);
  for (int d = tid; d < int(nb); d += kTopThreads) {
    uint32_t c = 0;
#pragma unroll 8
    for (int32_t b = 0; b < B; ++b) c += ghist[(int64_t(qh) * B + b) * 2048 + d];   // 8 loads in flight
    hist[d] = c;
  }
  const uint32_t prefix = pass ? state[4 * qh] : 0u, pmask = pass ? state[4 * qh + 1] : 0u;
  const uint32_t need = pass ? state[4 * qh + 2] : uint32_t(k);
  __syncthreads();
  uint32_t digit, above;
  block_find_digit<kTopThreads>(hist, nb, need, s_tmp, digit, above, &s_digit, &s_above);
  if (tid == 0) {
    state[4 * qh] = prefix | (digit << shift);
    state[4 * qh + 1] = pmask | ((nb - 1) << shift);
    state[4 * qh + 2] = need - above;
  }
}

// Keys of a segment above tau and equal to tau: cnt[(qh * B + b) * 2 + {0, 1}].
__global__ __launch_bounds__(kSegThreads) void topk_seg_count_kernel(const float* __restrict__ scores, int32_t T,
                                                                      int32_t B, int32_t S,
                                                                      const uint32_t* __restrict__ state,
                                                                      uint32_t* __restrict__ cnt) {
  __shared__ uint32_t s_cnt[kSegWaves][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t b = blockIdx.x, qh = blockIdx.y;
  const float* sc = scores + int64_t(qh) * score_stride(T);
  const uint32_t tau = state[4 * qh];
  const int32_t lo = b * S, hi = min(T, lo + S);
  uint32_t gt = 0, eq = 0;
  for (int32_t t0 = lo; t0 < hi; t0 += 4 * kSegThreads * kTopBatch) {
    uint32_t key[kTopBatch][4];
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) keys4(sc, t0 + 4 * (i * kSegThreads + tid), hi, key[i]);
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = t0 + 4 * (i * kSegThreads + tid) + e < hi;
        gt += in && key[i][e] > tau;
        eq += in && key[i][e] == tau;
      }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) { s_cnt[wave][0] = gt; s_cnt[wave][1] = eq; }
  __syncthreads();
  if (tid == 0) {
    uint32_t g = 0, q = 0;
    for (int w = 0; w < kSegWaves; ++w) { g += s_cnt[w][0]; q += s_cnt[w][1]; }
    cnt[(int64_t(qh) * B + b) * 2] = g;
    cnt[(int64_t(qh) * B + b) * 2 + 1] = q;
  }
}

// The segment's selected positions in position order: wave w of the block owns the contiguous
// part [lo + w*seg, lo + (w+1)*seg) of the segment, 256 positions per step (lane l holds
// positions 4l..4l+3 of the step), ranked with ballots as in topk_kernel.
__global__ __launch_bounds__(kSegThreads) void topk_seg_write_kernel(const float* __restrict__ scores, int32_t T,
                                                                      int32_t B, int32_t S, int32_t k,
                                                                      const uint32_t* __restrict__ state,
                                                                      const uint32_t* __restrict__ cnt,
                                                                      int32_t* __restrict__ sel) {
  __shared__ uint32_t s_cnt[kSegWaves][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  const int32_t b = blockIdx.x, qh = blockIdx.y;
  const float* sc = scores + int64_t(qh) * score_stride(T);
  const uint32_t tau = state[4 * qh], need = state[4 * qh + 2];
  uint32_t g_seg = 0, e_seg = 0;                          // earlier segments of the head
  for (int32_t c = 0; c < b; ++c) {
    g_seg += cnt[(int64_t(qh) * B + c) * 2];
    e_seg += cnt[(int64_t(qh) * B + c) * 2 + 1];
  }
  const int32_t seg_lo = b * S, seg_hi = min(T, seg_lo + S);
  const int32_t part = (((seg_hi - seg_lo) + kSegWaves - 1) / kSegWaves + 255) & ~255;
  const int32_t lo = min(seg_hi, seg_lo + wave * part), hi = min(seg_hi, lo + part);
  uint32_t gt = 0, eq = 0;
  for (int32_t t0 = lo; t0 < hi; t0 += 256 * kTopBatch) {
    uint32_t key[kTopBatch][4];
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) keys4(sc, t0 + 256 * i + 4 * lane, hi, key[i]);
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) {
      uint32_t g = 0, q = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = t0 + 256 * i + 4 * lane + e < hi;
        g += in && key[i][e] > tau;
        q += in && key[i][e] == tau;
      }
      gt += wave_sum(g);
      eq += wave_sum(q);
    }
  }
  if (lane == 0) { s_cnt[wave][0] = gt; s_cnt[wave][1] = eq; }
  __syncthreads();
  uint32_t g0 = g_seg, e0 = e_seg;
  for (int w = 0; w < wave; ++w) { g0 += s_cnt[w][0]; e0 += s_cnt[w][1]; }
  int32_t* dst = sel + int64_t(qh) * k;
  uint32_t out = g0 + min(e0, need), e_seen = e0;
  for (int32_t t0 = lo; t0 < hi; t0 += 256 * kTopBatch) {
    uint32_t key[kTopBatch][4];
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) keys4(sc, t0 + 256 * i + 4 * lane, hi, key[i]);
#pragma unroll
    for (int i = 0; i < kTopBatch; ++i) {
      const int32_t tb = t0 + 256 * i + 4 * lane;
      bool is_eq[4];
      uint32_t q = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        is_eq[e] = tb + e < hi && key[i][e] == tau;
        q += is_eq[e];
      }
      uint32_t eq_rank = e_seen + lanes_below_sum(q, below);
      bool take[4];
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        take[e] = (tb + e < hi && key[i][e] > tau) || (is_eq[e] && eq_rank < need);
        eq_rank += is_eq[e];
        c += take[e];
      }
      uint32_t slot = out + lanes_below_sum(c, below);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (take[e]) {
          if (slot < uint32_t(k)) dst[slot] = tb + e;
          ++slot;
        }
      out += wave_sum(c);
      e_seen += wave_sum(q);
    }
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
// A block covers 4 waves x kKeysPerWave keys of one query head, in 16-key slices.  Lane (n, kb) =
// (lane & 15, lane >> 4) holds key n of the slice, channels 32 kb .. 32 kb + 31; a key's score
// is summed over its 4 kb lanes, a slice's softmax over the 16 n lanes, and each lane
// accumulates its own 32 output channels.
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

// The K parameters of the lane's channels 32 kb .. 32 kb + 31 of one key: 16-byte chunks 8 kb ..
// 8 kb + 7 of the key's 512-byte row ((f16 scale, f16 zero) per channel), 128 contiguous bytes.
// Loaded lane by lane that would be 8 loads each touching 64 cache lines per wave; instead load i
// takes chunk 4 i + kb, so a key's 4 lanes read 64 contiguous bytes per load, and a 4 x 4
// transpose of 8-dword blocks across the 16-lane rows (permlane32 then permlane16 swaps) hands
// every lane its own chunks: afterwards e[r][0..3] is chunk 8 kb + r and e[r][4..7] chunk
// 8 kb + 4 + r.  All 4 lanes of a key take this path together or not at all.
__device__ __forceinline__ void k_params_row(const uint32_t* __restrict__ row, int kb, uint32_t e[4][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {                // block i / 2 is bound for row i / 2
    const uint4 v = *reinterpret_cast<const uint4*>(row + 4 * (4 * i + kb));
    uint32_t* d = &e[i >> 1][4 * (i & 1)];
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) {                // rows 2, 3 of blocks 0, 1 <-> rows 0, 1 of blocks 2, 3
    const auto a = __builtin_amdgcn_permlane32_swap(e[0][x], e[2][x], false, false);
    e[0][x] = a[0]; e[2][x] = a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(e[1][x], e[3][x], false, false);
    e[1][x] = b[0]; e[3][x] = b[1];
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) {                // odd rows of blocks 0, 2 <-> even rows of blocks 1, 3
    const auto a = __builtin_amdgcn_permlane16_swap(e[0][x], e[1][x], false, false);
    e[0][x] = a[0]; e[1][x] = a[1];
    const auto b = __builtin_amdgcn_permlane16_swap(e[2][x], e[3][x], false, false);
    e[2][x] = b[0]; e[3][x] = b[1];
  }
}

// The lane's 32 channels 32 kb .. 32 kb + 31 of key position p of KV head h at the chain's
// depth, as binary32 values that are exactly the BF16 reconstruction.  One 16-byte code load
// per loop (the four octets are contiguous); an INT4 V loop's group word is one load (the 32
// channels lie in one 64-channel group); INT4 K parameters through k_params_row.  The chain's
// sums bf16(acc) + bf16(d) go through v_dot2_f32_bf16 (add_rounded_bf16x8).  FMT: the chain's
// stream formats (INT4, or FP4 loops as the fused decode attention takes them).
template <int KIND, int NL, int FMT>
__device__ __forceinline__ void gather_row32(const ChainArgs& c, const int32_t* const* maps, int32_t p, int32_t H,
                                             int32_t h, int kb, uint32_t ones, float acc[32]) {
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    if (l >= c.n_loops) continue;
    const StreamArgs& st = c.s[l];
    const int32_t j = st.rows == nullptr ? p : maps[l][p];
    if (j < 0) continue;                                     // absent: inherits
    const uint32_t item = uint32_t(j) * uint32_t(H) + uint32_t(h);
    const uint4 cw4 = *reinterpret_cast<const uint4*>(st.codes + (item * (kSD / 2) + 16u * uint32_t(kb)));
    const uint32_t cws[4] = {cw4.x, cw4.y, cw4.z, cw4.w};
    uint32_t vw = 0;
    if (KIND == FLK_KIND_V && !loop_fp4<FMT>(l)) vw = st.params[item * 2u + uint32_t(kb >> 1)];
    // an FP4 loop's block scales of the lane's 32 channels, one load per loop: NVFP4 the E4M3
    // pair of blocks 2 kb, 2 kb + 1 (octets 0-1 and 2-3) times the stream scale, MXFP4 the E8M0
    // byte of block kb
    float fs[2] = {0.0f, 0.0f};
    if (loop_fp4<FMT>(l)) {
      const uint8_t* pb = reinterpret_cast<const uint8_t*>(st.params);
      if (loop_mx<FMT>(l)) {
        fs[0] = fs[1] = fp4_e8m0_value(pb[item * 4u + uint32_t(kb)]);
      } else {
        const fp4_f32x2 s2 = e4m3x2_value(*reinterpret_cast<const uint16_t*>(pb + 16u + item * 8u + 2u * uint32_t(kb)));
        const float gs = __uint_as_float(st.params[0]);
        fs[0] = s2.x * gs;
        fs[1] = s2.y * gs;
      }
    }
    uint32_t kp[4][8];
    if (KIND == FLK_KIND_K && !loop_fp4<FMT>(l)) {
      const uint32_t row = c.ktile ? uint32_t(p) / kGroup : uint32_t(j) / kGroup;
      k_params_row(st.params + (row * uint32_t(H) + uint32_t(h)) * kSD, kb, kp);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float d[8];
      if (loop_fp4<FMT>(l)) {
        fp4_decode8(cws[i], fs[i >> 1], d);
      } else {
        uint32_t pw[8];
        if (KIND == FLK_KIND_K) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {           // octet i: chunks 8 kb + 2 i and 8 kb + 2 i + 1
            pw[e] = kp[(2 * i) & 3][4 * (i >> 1) + e];
            pw[4 + e] = kp[(2 * i + 1) & 3][4 * (i >> 1) + e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pw[e] = vw;
        }
        float cv[8];
        codes8_to_f32(cws[i], cv);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = decode(cv[e], f16_bits_to_f32(pw[e] & 0xFFFFu), f16_bits_to_f32(pw[e] >> 16));
      }
      float* a8 = acc + 8 * i;
      if (l == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] = d[e];
      } else {
        add_rounded_bf16x8(a8, d, ones);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) round_bf16x8(acc + 8 * i);   // the last rounding, in place
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
template <int NL, int MODE, int FMT>
__global__ __launch_bounds__(kSThreads) void sparse_gather_kernel(GatherArgs g) {
  __shared__ float s_m[kSWaves], s_l[kSWaves];
  __shared__ float s_o[kSWaves][kSD];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int32_t qh = blockIdx.y, h = qh / g.G;
  const int32_t key0 = int32_t(blockIdx.x) * kKeysPerBlock + wave * kKeysPerWave;
  const int32_t* sel = g.sel + int64_t(qh) * g.k;

  // the query's channels 32 kb .. 32 kb + 31 as BF16 pairs (the score is a sum of dot2 steps)
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  uint32_t qp[16];
  if (MODE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(g.q + int64_t(qh) * kSD + 32 * kb + 8 * i);
      qp[4 * i + 0] = w.x; qp[4 * i + 1] = w.y; qp[4 * i + 2] = w.z; qp[4 * i + 3] = w.w;
    }
  }
  const uint32_t ones = bf16_ones();
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
        float kv[32];
        gather_row32<FLK_KIND_K, NL, FMT>(g.kc, g.kmap, p, g.H, h, kb, ones, kv);
#pragma unroll
        for (int c2 = 0; c2 < 16; ++c2)                   // K_hat is exactly BF16: the pairs are exact
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pack_bf16x2(kv[2 * c2], kv[2 * c2 + 1])),
                                              __builtin_bit_cast(bf16x2v, qp[c2]), s, false);
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
        float vv[32];
        gather_row32<FLK_KIND_V, NL, FMT>(g.vc, g.vmap, p, g.H, h, kb, ones, vv);
#pragma unroll
        for (int c2 = 0; c2 < 32; ++c2) o[c2] = __builtin_fmaf(pn, vv[c2], o[c2]);
      }
    } else {
      const float w = p >= 0 ? __expf(g.scores[int64_t(qh) * score_stride(g.T) + p] - M) * Linv : 0.0f;
      m_run += sum16(w);
      if (p >= 0) {
        float vv[32];
        gather_row32<FLK_KIND_V, NL, FMT>(g.vc, g.vmap, p, g.H, h, kb, ones, vv);
#pragma unroll
        for (int c2 = 0; c2 < 32; ++c2) o[c2] = __builtin_fmaf(w, vv[c2], o[c2]);
      }
    }
  }
  // this wave's output channels: sum over the 16 keys of the slice lanes
#pragma unroll
  for (int c = 0; c < 32; ++c) o[c] = sum16(o[c]);
  if (n == 0) {
#pragma unroll
    for (int c2 = 0; c2 < 32; ++c2) s_o[wave][32 * kb + c2] = o[c2];
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

// Per query head (block): merge the gather blocks' partials.  Thread (grp, c) = (tid / 128,
// tid % 128) folds channel c of the blocks grp, grp + kCombGroups, ..., kCombBatch of them per
// batch of loads (nblk <= kCombGroups * kCombBatch is one batch), and the groups' folds merge
// through LDS.  MODE 0: mass[qh] = sum of masses, c_ref[qh][c] = sum.  MODE 1: out = O_ref -
// C_ref + m * o / l, the partials (max, sum, o) merged as in an online softmax.
constexpr int kCombGroups = 8;
constexpr int kCombBatch = 8;
template <int MODE>
__global__ __launch_bounds__(kCombGroups * kSD) void sparse_combine_kernel(
    const float* __restrict__ part, int32_t nblk, float* __restrict__ mass_out, float* __restrict__ c_out,
    const float* __restrict__ mass, const float* __restrict__ o_ref, const float* __restrict__ c_ref,
    uint16_t* __restrict__ out) {
  __shared__ float s_m[kCombGroups], s_l[kCombGroups];
  __shared__ float s_o[kCombGroups][kSD];
  const int32_t qh = blockIdx.x;
  const int c = threadIdx.x % kSD, grp = threadIdx.x / kSD;
  const float* pp = part + int64_t(qh) * nblk * (2 + kSD);
  float M = MODE == 1 ? -__builtin_inff() : 0.0f;           // mode 0: the mass
  float L = 0.0f, O = 0.0f;
  for (int32_t b0 = grp; b0 < nblk; b0 += kCombGroups * kCombBatch) {
    float mb[kCombBatch], lb[kCombBatch], ob[kCombBatch];
#pragma unroll
    for (int i = 0; i < kCombBatch; ++i) {
      const int32_t b = b0 + i * kCombGroups;
      const bool ok = b < nblk;
      mb[i] = ok ? pp[b * (2 + kSD)] : (MODE == 1 ? -__builtin_inff() : 0.0f);
      lb[i] = ok && MODE == 1 ? pp[b * (2 + kSD) + 1] : 0.0f;
      ob[i] = ok ? pp[b * (2 + kSD) + 2 + c] : 0.0f;
    }
    if (MODE == 0) {
#pragma unroll
      for (int i = 0; i < kCombBatch; ++i) {
        M += mb[i];
        O += ob[i];
      }
    } else {
      float mx = M;
#pragma unroll
      for (int i = 0; i < kCombBatch; ++i) mx = fmaxf(mx, mb[i]);
      const float f0 = M == -__builtin_inff() ? 0.0f : __expf(M - mx);
      L *= f0;
      O *= f0;
#pragma unroll
      for (int i = 0; i < kCombBatch; ++i) {
        const float f = mb[i] == -__builtin_inff() ? 0.0f : __expf(mb[i] - mx);
        L += lb[i] * f;
        O += ob[i] * f;
      }
      M = mx;
    }
  }
  s_o[grp][c] = O;
  if (c == 0) {
    s_m[grp] = M;
    s_l[grp] = L;
  }
  __syncthreads();
  if (grp != 0) return;
  if (MODE == 0) {
#pragma unroll
    for (int i = 1; i < kCombGroups; ++i) {
      O += s_o[i][c];
      M += s_m[i];
    }
    c_out[int64_t(qh) * kSD + c] = O;
    if (c == 0) mass_out[qh] = M;
  } else {
#pragma unroll
    for (int i = 1; i < kCombGroups; ++i) M = fmaxf(M, s_m[i]);
    L = 0.0f;
    O = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombGroups; ++i) {
      const float f = s_m[i] == -__builtin_inff() ? 0.0f : __expf(s_m[i] - M);
      L += s_l[i] * f;
      O += s_o[i][c] * f;
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
  size_t kmaps, vmaps, part, attn, scores, ml, topk, total;
};
static SparseLayout sparse_layout(int32_t T, int32_t H, int32_t Hq, int32_t k, int32_t n_loops) {
  SparseLayout L{};
  size_t off = 0;
  const size_t map_bytes = align256(size_t(T) * sizeof(int32_t)) * size_t(n_loops);
  L.kmaps = off; off += map_bytes;
  L.vmaps = off; off += map_bytes;
  L.part = off; off += align256(size_t(Hq) * gather_blocks(k) * (2 + kSD) * sizeof(float));
  L.attn = off; off += align256(attn_workspace_bytes(T, H, Hq));
  L.scores = off; off += align256(size_t(Hq) * size_t(score_stride(T)) * sizeof(float));
  L.ml = off; off += align256(size_t(Hq) * 2 * sizeof(float));
  L.topk = off;                                  // split top-k: state, segment counts, histograms
  if (T > kSplitMinT) {
    const SplitTopk st = split_topk(T);
    off += align256(size_t(Hq) * 4 * sizeof(uint32_t)) + align256(size_t(Hq) * st.B * 2 * sizeof(uint32_t)) +
           align256(size_t(Hq) * st.B * 2048 * sizeof(uint32_t));
  }
  L.total = off;
  return L;
}

size_t sparse_workspace_bytes(int32_t T, int32_t H, int32_t Hq, int32_t k, int32_t n_loops) {
  return sparse_layout(T, H, Hq, k, n_loops).total;
}

// One launch builds the maps of every compact loop of both chains.  A V loop that shares its
// rows and tile index with a K loop (one selection stored once) reuses the K loop's map.
static hipError_t build_maps(const ChainArgs* kc, const ChainArgs& vc, int32_t T, int32_t* kbase, int32_t* vbase,
                             const int32_t** kmaps, const int32_t** vmaps, hipStream_t stream) {
  MapJobs jobs{};
  jobs.T = T;
  const size_t stride = align256(size_t(T) * sizeof(int32_t)) / sizeof(int32_t);
  for (int l = 0; l < FLK_MAX_LOOPS; ++l) kmaps[l] = vmaps[l] = nullptr;
  if (kc != nullptr) {
    for (int l = 0; l < kc->n_loops; ++l) {
      if (kc->s[l].rows == nullptr) continue;
      int32_t* m = kbase + size_t(l) * stride;
      jobs.j[jobs.n_jobs++] = MapJob{kc->s[l].rows, kc->s[l].tile_start, m, kc->s[l].n};
      kmaps[l] = m;
    }
  }
  for (int l = 0; l < vc.n_loops; ++l) {
    if (vc.s[l].rows == nullptr) continue;
    for (int i = 0; i < jobs.n_jobs && vmaps[l] == nullptr; ++i)
      if (jobs.j[i].rows == vc.s[l].rows && jobs.j[i].tile_start == vc.s[l].tile_start && jobs.j[i].n == vc.s[l].n)
        vmaps[l] = jobs.j[i].map;
    if (vmaps[l] != nullptr) continue;
    int32_t* m = vbase + size_t(l) * stride;
    jobs.j[jobs.n_jobs++] = MapJob{vc.s[l].rows, vc.s[l].tile_start, m, vc.s[l].n};
    vmaps[l] = m;
  }
  if (jobs.n_jobs == 0) return hipSuccess;
  const int32_t ntiles = (T + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(chain_map_kernel, dim3(unsigned((ntiles + kSWaves - 1) / kSWaves), unsigned(jobs.n_jobs)),
                     dim3(kSThreads), 0, stream, jobs);
  return hipGetLastError();
}

template <int MODE, int FMT>
static hipError_t launch_gather_fmt(const GatherArgs& g, int nl, hipStream_t stream) {
  const dim3 grid(unsigned(g.nblk), unsigned(g.H * g.G));
#define FLK_G(NLV)                                                                                        \
  case NLV:                                                                                               \
    hipLaunchKernelGGL((sparse_gather_kernel<NLV, MODE, FMT>), grid, dim3(kSThreads), 0, stream, g);    \
    break;
  switch (nl) {
    FLK_G(1) FLK_G(2) FLK_G(3) FLK_G(4) FLK_G(5) FLK_G(6) FLK_G(7) FLK_G(8)
    default: return hipErrorInvalidValue;
  }
#undef FLK_G
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gather(const GatherArgs& g, int nl, int fmt, hipStream_t stream) {
  switch (fmt) {
    case 0: return launch_gather_fmt<MODE, 0>(g, nl, stream);
    case 1: return launch_gather_fmt<MODE, 1>(g, nl, stream);
    case 2: return launch_gather_fmt<MODE, 2>(g, nl, stream);
    case 3: return launch_gather_fmt<MODE, 3>(g, nl, stream);
    case 4: return launch_gather_fmt<MODE, 4>(g, nl, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sparse_reference(int fmt, int32_t T, int32_t H, int32_t Hq, int32_t k, const void* q,
                                   const ChainArgs& kc, const ChainArgs& vc, float scale, void* out, int32_t* sel,
                                   float* mass, float* o_ref, float* c_ref, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  const int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  const SparseLayout L = sparse_layout(T, H, Hq, k, nl);
  if (ws == nullptr || ws_bytes < L.total || k < 1 || k > T) return hipErrorInvalidValue;
  char* w = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(w + L.scores);
  float* ml = reinterpret_cast<float*>(w + L.ml);
  hipError_t e = launch_attn_reference(fmt, T, H, Hq, q, kc, vc, scale, out, o_ref, ml, scores, w + L.attn,
                                       attn_workspace_bytes(T, H, Hq), stream);
  if (e != hipSuccess) return e;
  if (T > kSplitMinT) {
    const SplitTopk st = split_topk(T);
    uint32_t* state = reinterpret_cast<uint32_t*>(w + L.topk);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(w + L.topk + align256(size_t(Hq) * 4 * sizeof(uint32_t)));
    uint32_t* ghist = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(cnt) +
                                                  align256(size_t(Hq) * st.B * 2 * sizeof(uint32_t)));
    const dim3 sgrid(unsigned(st.B), unsigned(Hq));
    for (int pass = 0; pass < 3; ++pass) {
      hipLaunchKernelGGL(topk_seg_hist_kernel, sgrid, dim3(kSegThreads), 0, stream, scores, T, st.B, st.S, pass,
                         state, ghist);
      hipLaunchKernelGGL(topk_seg_digit_kernel, dim3(unsigned(Hq)), dim3(kTopThreads), 0, stream, st.B, k, pass,
                         ghist, state);
    }
    hipLaunchKernelGGL(topk_seg_count_kernel, sgrid, dim3(kSegThreads), 0, stream, scores, T, st.B, st.S, state,
                       cnt);
    hipLaunchKernelGGL(topk_seg_write_kernel, sgrid, dim3(kSegThreads), 0, stream, scores, T, st.B, st.S, k, state,
                       cnt, sel);
  } else {
    hipLaunchKernelGGL(topk_kernel, dim3(unsigned(Hq)), dim3(kTopThreads), 0, stream, scores, T, k, sel);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  GatherArgs g{};
  g.kc = kc;
  g.vc = vc;
  if ((e = build_maps(nullptr, vc, T, nullptr, reinterpret_cast<int32_t*>(w + L.vmaps), g.kmap, g.vmap, stream)) !=
      hipSuccess)
    return e;
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
  if ((e = launch_gather<0>(g, vc.n_loops, fmt, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_combine_kernel<0>), dim3(unsigned(Hq)), dim3(kCombGroups * kSD), 0, stream, g.part,
                     g.nblk, mass, c_ref, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_sparse_loop(int fmt, int32_t T, int32_t H, int32_t Hq, int32_t k, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, float scale, const int32_t* sel,
                              const float* mass, const float* o_ref, const float* c_ref, void* out, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  const int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  const SparseLayout L = sparse_layout(T, H, Hq, k, nl);
  if (ws == nullptr || ws_bytes < L.part + align256(size_t(Hq) * gather_blocks(k) * (2 + kSD) * sizeof(float)) ||
      k < 1 || k > T)
    return hipErrorInvalidValue;
  char* w = static_cast<char*>(ws);
  GatherArgs g{};
  g.kc = kc;
  g.vc = vc;
  hipError_t e = build_maps(&kc, vc, T, reinterpret_cast<int32_t*>(w + L.kmaps),
                            reinterpret_cast<int32_t*>(w + L.vmaps), g.kmap, g.vmap, stream);
  if (e != hipSuccess) return e;
  g.q = static_cast<const uint16_t*>(q);
  g.sel = sel;
  g.part = reinterpret_cast<float*>(w + L.part);
  g.T = T;
  g.H = H;
  g.G = Hq / H;
  g.k = k;
  g.nblk = gather_blocks(k);
  g.scale = scale;
  if ((e = launch_gather<1>(g, nl, fmt, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL((sparse_combine_kernel<1>), dim3(unsigned(Hq)), dim3(kCombGroups * kSD), 0, stream, g.part,
                     g.nblk, nullptr, nullptr, mass, o_ref, c_ref, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace flk
