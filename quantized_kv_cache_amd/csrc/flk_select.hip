// flk_select.hip -- token selection for sparse prefill (FlashLoop integration RFC, vllm-rlt
// issue #156, section 3.1 "Token-sparse prefill" with its fixed selection windows) and the
// stable partition of a submission's rows (section 6.2).
//
//   score_kernel        one wave per eligible token: both norms of the change score, with each
//                       sum of squares in pairwise order over the channel index
//   window_count_kernel one workgroup: every window's budget (capped by its eligible tokens)
//                       and their exclusive prefix, i.e. where each window's rows start
//   window_topk_kernel  one workgroup per window: radix select of the budget's threshold
//                       score, then the window's selected positions in position order
//   partition_kernel    one workgroup: decode rows, then active prefill rows, stably
#include <hip/hip_runtime.h>

#include <cstdint>

#include "flk_blockscan.h"
#include "flk_device.h"
#include "flk_internal.h"
#include "flk_select.h"

namespace flk {

namespace {

// ---------------------------------------------------------------------------------------
// Change scores.  Lane l of the wave reads channels 512c + 8l .. 512c + 8l + 7 of chunk c
// (16 coalesced bytes per lane and tensor).  The pairwise tree over the channel index is
// then: the 8 channels of a lane (levels 1-3), the 64 lanes of a chunk (levels 4-9), the
// chunks (levels 10 and up).  Levels 4-9 run as a reduce-scatter over the chunks: at lane bit
// s each lane keeps half of its chunks and adds the partner's partial sums of that half, so
// after log2(chunks) steps a lane holds one chunk (index = its low bits reversed) and the last
// levels are plain butterflies.  Each addition adds two sibling subtrees, and binary32
// addition is commutative, so every lane computes exactly the tree's value.
// ---------------------------------------------------------------------------------------
constexpr int kScoreWaves = 4;
constexpr int kMaxChunks = 32;               // d <= 16384
constexpr int kChunkBatch = 8;               // chunks loaded per batch (16 loads in flight)
constexpr int kRowsPerWave = 4;

__device__ __forceinline__ float tree8(const float v[8]) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

// Squares of h1 - h2 and of h1 over one lane's 8 channels, summed pairwise.
__device__ __forceinline__ void lane_sums(const uint4& a, const uint4& b, float& num, float& den) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
  float sq[8], aa[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a0 = __uint_as_float(wa[i] << 16), a1 = __uint_as_float(wa[i] & 0xFFFF0000u);
    const float b0 = __uint_as_float(wb[i] << 16), b1 = __uint_as_float(wb[i] & 0xFFFF0000u);
    const float d0 = a0 - b0, d1 = a1 - b1;
    sq[2 * i] = d0 * d0;
    sq[2 * i + 1] = d1 * d1;
    aa[2 * i] = a0 * a0;
    aa[2 * i + 1] = a1 * a1;
  }
  num = tree8(sq);
  den = tree8(aa);
}

template <int P>
__device__ __forceinline__ int bitrev(int x) {
  int r = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) r |= ((x >> i) & 1) << (P - 1 - i);
  return r;
}

// v[0..2^P) per lane (chunk partial sums) -> the tree sum over all chunks and lanes, in every lane.
template <int P>
__device__ __forceinline__ float wave_tree(float v[1 << P], int lane) {
  constexpr int NC = 1 << P;
#pragma unroll
  for (int s = 0; s < P; ++s) {
    const bool up = (lane >> s) & 1;
    const int half = NC >> (s + 1);
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = up ? v[i] : v[i + half];
      const float keep = up ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, 1 << s);
    }
  }
#pragma unroll
  for (int s = P; s < 6; ++s) v[0] += __shfl_xor(v[0], 1 << s);
  float c[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) c[i] = __shfl(v[0], bitrev<P>(i));
#pragma unroll
  for (int len = NC; len > 1; len >>= 1)
#pragma unroll
    for (int i = 0; i < len / 2; ++i) c[i] = c[2 * i] + c[2 * i + 1];
  return c[0];
}

// A wave scores rows wid, wid + nw, wid + 2nw, ... (nw waves in the grid).  The loads of the
// next batch of chunks (the next row's first batch after a row's last) are issued before the
// current row's cross-lane tree, so every wave keeps a row's bytes in flight while it reduces.
template <int P>
__global__ __launch_bounds__(64 * kScoreWaves) void score_kernel(const uint16_t* __restrict__ h1,
                                                                  const uint16_t* __restrict__ h2, int32_t d,
                                                                  const int32_t* __restrict__ rows, int32_t n,
                                                                  float eps, float* __restrict__ scores,
                                                                  uint32_t* __restrict__ status) {
  constexpr int NC = 1 << P;
  constexpr int B = NC < kChunkBatch ? NC : kChunkBatch;   // chunks per batch of loads
  constexpr int NB = NC / B;                                // batches per row
  const int lane = threadIdx.x & 63;
  const int32_t wid = blockIdx.x * kScoreWaves + int32_t(threadIdx.x >> 6);
  const int32_t nw = gridDim.x * kScoreWaves;
  if (wid >= n) return;                                     // whole waves; no workgroup barrier below
  const int32_t my_rows = (n - 1 - wid) / nw + 1;
  uint4 va[B], vb[B];
  auto issue = [&](int32_t r, int bt) {
    const int32_t j = wid + r * nw;
    const int64_t p = rows ? rows[j] : j;
    const uint16_t* a = h1 + p * d;
    const uint16_t* b = h2 + p * d;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int32_t ch = 512 * (bt * B + i) + 8 * lane;
      if (ch < d) {
        va[i] = *reinterpret_cast<const uint4*>(a + ch);
        vb[i] = *reinterpret_cast<const uint4*>(b + ch);
      } else {
        va[i] = make_uint4(0, 0, 0, 0);
        vb[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  issue(0, 0);
  for (int32_t r = 0; r < my_rows; ++r) {
    float num[NC], den[NC];
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
#pragma unroll
      for (int i = 0; i < B; ++i) lane_sums(va[i], vb[i], num[bt * B + i], den[bt * B + i]);
      // keep the next loads after this batch's arithmetic: hoisting them would hold two
      // batches of loaded data in registers
      __builtin_amdgcn_sched_barrier(0);
      if (bt + 1 < NB) issue(r, bt + 1);
      else if (r + 1 < my_rows) issue(r + 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float sn = wave_tree<P>(num, lane);
    const float sd = wave_tree<P>(den, lane);
    if (lane == 0) {
      const float s = __builtin_sqrtf(sn) / __builtin_fmaxf(__builtin_sqrtf(sd), eps);
      scores[wid + r * nw] = s;
      if (status && !__builtin_isfinite(s)) atomicOr(status, FLK_DEV_NONFINITE);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Window budgets and where each window's rows start.
// ---------------------------------------------------------------------------------------
constexpr int kCountThreads = 1024;

__device__ __forceinline__ int32_t lower_bound_seq(const int32_t* __restrict__ rows, int32_t n, int64_t key) {
  int32_t a = 0, b = n;
  while (a < b) {
    const int32_t m = (a + b) >> 1;
    if (rows[m] < key) a = m + 1; else b = m;
  }
  return a;
}

__device__ __forceinline__ int32_t window_take(const int32_t* rows, int32_t n_prev, int32_t T, int32_t window,
                                               int32_t pct, int32_t w) {
  const int64_t w0 = int64_t(w) * window;
  const int64_t len = (w0 + window <= T) ? window : T - w0;
  const int64_t elig = rows ? lower_bound_seq(rows, n_prev, w0 + len) - lower_bound_seq(rows, n_prev, w0) : len;
  const int64_t budget = (int64_t(pct) * len + 99) / 100;
  return int32_t(budget < elig ? budget : elig);
}

__global__ __launch_bounds__(kCountThreads) void window_count_kernel(const int32_t* __restrict__ rows, int32_t n_prev,
                                                                      int32_t T, int32_t window, int32_t pct,
                                                                      int32_t n_win, int32_t n_out,
                                                                      int32_t* __restrict__ offs,
                                                                      uint32_t* __restrict__ status) {
  __shared__ int32_t wsum[kCountThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t run = 0;
  for (int32_t base = 0; base < n_win; base += kCountThreads) {
    const int32_t w = base + tid;
    const int32_t k = w < n_win ? window_take(rows, n_prev, T, window, pct, w) : 0;
    int32_t inc = k;                                   // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int32_t before = 0, total = 0;
    for (int v = 0; v < kCountThreads / 64; ++v) {
      before += v < wave ? wsum[v] : 0;
      total += wsum[v];
    }
    if (w < n_win) offs[w] = run + before + inc - k;
    run += total;
    __syncthreads();
  }
  if (tid == 0) {
    offs[n_win] = run;
    if (run != n_out && status) atomicOr(status, FLK_DEV_COUNT);
  }
}

// ---------------------------------------------------------------------------------------
// Per-window top-k.  The window's eligible tokens are a contiguous run [lo, hi) of the score
// array.  A radix select over order-preserving keys of the scores (digits of 11, 11 and 10
// bits) finds the k-th largest key tau and how many keys equal to tau are taken (the lowest
// positions first); a pass in position order then writes the selected positions, a block's
// width at a time, ranked with ballots.
//
// With at most kWinThreads windows (OWN), each block finds where every window's run starts from
// one pass over the eligible list (no atomics: the list is ascending) and scans the budgets
// itself; otherwise window_count_kernel has written the budgets' prefix and the run is found
// by two searches (block_lower_bound probes with the first 256 threads of the block).
// ---------------------------------------------------------------------------------------
constexpr int kWinThreads = 1024;
constexpr int kCacheKeys = 4;                // keys per thread kept in registers

__device__ __forceinline__ uint32_t sel_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool OWN>
__global__ __launch_bounds__(kWinThreads) void window_topk_kernel(const float* __restrict__ scores,
                                                                   const int32_t* __restrict__ rows, int32_t n_prev,
                                                                   int32_t T, int32_t window, int32_t pct,
                                                                   int32_t n_win, const int32_t* __restrict__ offs,
                                                                   int32_t n_out, int32_t* __restrict__ rows_out,
                                                                   int32_t* __restrict__ slot,
                                                                   uint32_t* __restrict__ status) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_digit, s_above;
  __shared__ int32_t s_wave[kWinThreads / 64][2];
  __shared__ int32_t s_run[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t w = blockIdx.x;
  const int64_t w0 = int64_t(w) * window;
  const int32_t len = int32_t((w0 + window <= T) ? window : T - w0);
  int32_t lo, hi, off, k;
  if (OWN) {
    // start[u] = the first eligible index at or past window u's first position; the list is
    // ascending, so entry i starts the windows after its predecessor's, up to its own
    int32_t* start = reinterpret_cast<int32_t*>(hist);  // n_win + 1 <= kWinThreads + 1 entries
    int32_t* tmp = &s_wave[0][0];
    for (int32_t u = tid; u <= n_win; u += kWinThreads)
      start[u] = rows ? n_prev : int32_t(min(int64_t(u) * window, int64_t(T)));
    __syncthreads();
    if (rows) {
      for (int32_t i = tid; i < n_prev; i += kWinThreads) {
        const int32_t v = min(max(rows[i], 0), T - 1) / window;
        const int32_t vp = i > 0 ? min(max(rows[i - 1], 0), T - 1) / window : -1;
        for (int32_t u = vp + 1; u <= v; ++u) start[u] = i;
      }
    }
    __syncthreads();
    int32_t e = 0, kt = 0;
    if (tid < n_win) {
      const int64_t lt = min(int64_t(window), int64_t(T) - int64_t(tid) * window);
      e = max(start[tid + 1] - start[tid], 0);
      kt = int32_t(min((int64_t(pct) * lt + 99) / 100, int64_t(e)));
    }
    int32_t tot_k;
    const int32_t ex_k = block_excl_scan<kWinThreads>(kt, tmp, tot_k);
    if (tid == w) { s_run[0] = start[w]; s_run[1] = e; s_run[2] = ex_k; s_run[3] = kt; }
    if (w == 0 && tid == 0 && tot_k != n_out && status) atomicOr(status, FLK_DEV_COUNT);
    __syncthreads();
    lo = min(max(s_run[0], 0), n_prev);
    hi = min(lo + s_run[1], n_prev);
    off = s_run[2];
    k = s_run[3];
  } else {
    lo = rows ? block_lower_bound(rows, n_prev, int32_t(w0)) : int32_t(w0);
    hi = rows ? block_lower_bound(rows, n_prev, int32_t(w0 + len)) : int32_t(w0 + len);
    off = offs[w];
    k = offs[w + 1] - off;                           // <= hi - lo by construction
  }
  if (slot) {
    for (int32_t p = tid; p < len; p += kWinThreads) slot[w0 + p] = -1;
    __syncthreads();                                   // before the selected entries overwrite them
  }
  if (k <= 0) return;
  const bool all = k >= hi - lo;
  // A run of at most kCacheKeys * kWinThreads keys is read once into registers (key r of a
  // thread is element lo + r * kWinThreads + tid); a longer one is re-read from memory.
  const bool cached = hi - lo <= kCacheKeys * kWinThreads;
  uint32_t kreg[kCacheKeys];
  if (cached && !all) {
#pragma unroll
    for (int r = 0; r < kCacheKeys; ++r) {
      const int32_t i = lo + r * kWinThreads + tid;
      kreg[r] = i < hi ? sel_key(scores[i]) : 0u;
    }
  }
  uint32_t tau = 0, need = 0;
  if (!all) {
    uint32_t prefix = 0, pmask = 0;
    need = uint32_t(k);
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
      const uint32_t nb = pass == 2 ? 1024u : 2048u;
      for (int b = tid; b < 2048; b += kWinThreads) hist[b] = 0;
      __syncthreads();
      if (cached) {
#pragma unroll
        for (int r = 0; r < kCacheKeys; ++r)
          if (lo + r * kWinThreads + tid < hi && (kreg[r] & pmask) == prefix)
            atomicAdd(&hist[(kreg[r] >> shift) & (nb - 1)], 1u);
      } else {
        for (int32_t i = lo + tid; i < hi; i += kWinThreads) {
          const uint32_t key = sel_key(scores[i]);
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
        }
      }
      __syncthreads();
      uint32_t digit, above;
      block_find_digit<kWinThreads>(hist, nb, need, &s_wave[0][0], digit, above, &s_digit, &s_above);
      prefix |= digit << shift;
      pmask |= (nb - 1) << shift;
      need -= above;
      __syncthreads();
    }
    tau = prefix;
  }
  // Position-ordered pass, a block's width of elements per step: element i of the run is taken
  // if all, or its key is above tau, or it is among the first `need` keys equal to tau.
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int32_t taken = 0, eq_seen = 0;
  auto step = [&](int32_t i, bool gt, bool eq) {
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) { s_wave[wave][0] = __builtin_popcountll(bg); s_wave[wave][1] = __builtin_popcountll(be); }
    __syncthreads();
    int32_t g_before = 0, e_before = 0, g_all = 0, e_all = 0;
    for (int v = 0; v < kWinThreads / 64; ++v) {
      g_before += v < wave ? s_wave[v][0] : 0;
      e_before += v < wave ? s_wave[v][1] : 0;
      g_all += s_wave[v][0];
      e_all += s_wave[v][1];
    }
    const int32_t e_rank = eq_seen + e_before + __builtin_popcountll(be & below);
    if (gt || (eq && e_rank < int32_t(need))) {
      // selected before this element in the run: those of earlier steps, the greater keys
      // before it in this step, and the equal keys before it that are among the first `need`
      const int32_t gt_before = g_before + __builtin_popcountll(bg & below);
      const int32_t r = off + taken + gt_before + min(e_rank, int32_t(need)) - min(eq_seen, int32_t(need));
      const int32_t pos = rows ? rows[i] : i;
      if (r < n_out) {
        rows_out[r] = pos;
        if (slot && pos >= 0 && pos < T) slot[pos] = r;
      }
    }
    taken += g_all + min(eq_seen + e_all, int32_t(need)) - min(eq_seen, int32_t(need));
    eq_seen += e_all;
    __syncthreads();
  };
  if (cached && !all) {
#pragma unroll
    for (int r = 0; r < kCacheKeys; ++r) {
      const int32_t base = lo + r * kWinThreads;
      if (base >= hi) break;                           // uniform over the block
      const bool in = base + tid < hi;
      step(base + tid, in && kreg[r] > tau, in && kreg[r] == tau);
    }
  } else {
    for (int32_t base = lo; base < hi; base += kWinThreads) {
      const int32_t i = base + tid;
      bool gt = false, eq = false;
      if (i < hi) {
        if (all) {
          gt = true;
        } else {
          const uint32_t key = sel_key(scores[i]);
          gt = key > tau;
          eq = key == tau;
        }
      }
      step(i, gt, eq);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Stable partition of execution rows: one workgroup; 4 rows per thread per step.
// ---------------------------------------------------------------------------------------
constexpr int kPartThreads = 1024;
constexpr int kPartRows = 4 * kPartThreads;

__global__ __launch_bounds__(kPartThreads) void partition_kernel(const uint8_t* __restrict__ cls, int32_t n,
                                                                  int32_t* __restrict__ gather,
                                                                  int32_t* __restrict__ scatter,
                                                                  int32_t* __restrict__ counts,
                                                                  uint32_t* __restrict__ status) {
  __shared__ int32_t tmp[kPartThreads / 64];
  const int tid = threadIdx.x;
  int32_t n_dec = 0;                                   // pass 1: decode rows in all
  for (int32_t base = 0; base < n; base += kPartRows) {
    int32_t c = 0;
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t i = base + 4 * tid + e;
      if (i < n) {
        const uint8_t v = cls[i];
        c += v == FLK_ROW_DECODE;
        bad |= v > FLK_ROW_DECODE;
      }
    }
    if (bad && status) atomicOr(status, FLK_DEV_CLASS);
    int32_t total;
    block_excl_scan<kPartThreads>(c, tmp, total);
    n_dec += total;
  }
  int32_t run_d = 0, run_a = 0;                        // pass 2: ranks and writes
  for (int32_t base = 0; base < n; base += kPartRows) {
    uint8_t v[4];
    int32_t cd = 0, ca = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t i = base + 4 * tid + e;
      v[e] = i < n ? cls[i] : uint8_t(FLK_ROW_INACTIVE);
      cd += v[e] == FLK_ROW_DECODE;
      ca += v[e] == FLK_ROW_ACTIVE;
    }
    int32_t td, ta;
    int32_t rd = run_d + block_excl_scan<kPartThreads>(cd, tmp, td);
    int32_t ra = n_dec + run_a + block_excl_scan<kPartThreads>(ca, tmp, ta);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t i = base + 4 * tid + e;
      if (i >= n) break;
      int32_t g = -1;
      if (v[e] == FLK_ROW_DECODE) g = rd++;
      else if (v[e] == FLK_ROW_ACTIVE) g = ra++;
      scatter[i] = g;
      if (g >= 0) gather[g] = i;
    }
    run_d += td;
    run_a += ta;
  }
  for (int32_t i = n_dec + run_a + tid; i < n; i += kPartThreads) gather[i] = -1;
  if (tid == 0) {
    counts[0] = n_dec;
    counts[1] = n_dec + run_a;
  }
}

}  // namespace

int32_t select_windows(int32_t T, int32_t window) { return int32_t((int64_t(T) + window - 1) / window); }

size_t select_workspace_bytes(int32_t T, int32_t window) {
  return (size_t(4) * (size_t(select_windows(T, window)) + 1) + 255) & ~size_t(255);
}

hipError_t launch_select_rows(const void* h_prev, const void* h_prev2, int32_t T, int32_t d, const int32_t* rows_prev,
                              int32_t n_prev, int32_t window, int32_t pct, float eps, float* scores,
                              int32_t* rows_out, int32_t n_out, int32_t* slot, void* ws, size_t ws_bytes,
                              uint32_t* status, hipStream_t stream) {
  const int32_t n_win = select_windows(T, window);
  if (ws == nullptr || ws_bytes < select_workspace_bytes(T, window) || d < 8 || d % 8 || d > 512 * kMaxChunks)
    return hipErrorInvalidValue;
  int32_t* offs = static_cast<int32_t*>(ws);
  if (pct > 0 && pct < 100 && n_prev > 0) {
    const auto* a = static_cast<const uint16_t*>(h_prev);
    const auto* b = static_cast<const uint16_t*>(h_prev2);
    const int32_t per_block = kScoreWaves * kRowsPerWave;
    const dim3 grid(unsigned((n_prev + per_block - 1) / per_block)), block(64 * kScoreWaves);
    const int chunks = (d + 511) / 512;
    if (chunks <= 1)
      hipLaunchKernelGGL(score_kernel<0>, grid, block, 0, stream, a, b, d, rows_prev, n_prev, eps, scores, status);
    else if (chunks <= 2)
      hipLaunchKernelGGL(score_kernel<1>, grid, block, 0, stream, a, b, d, rows_prev, n_prev, eps, scores, status);
    else if (chunks <= 4)
      hipLaunchKernelGGL(score_kernel<2>, grid, block, 0, stream, a, b, d, rows_prev, n_prev, eps, scores, status);
    else if (chunks <= 8)
      hipLaunchKernelGGL(score_kernel<3>, grid, block, 0, stream, a, b, d, rows_prev, n_prev, eps, scores, status);
    else if (chunks <= 16)
      hipLaunchKernelGGL(score_kernel<4>, grid, block, 0, stream, a, b, d, rows_prev, n_prev, eps, scores, status);
    else
      hipLaunchKernelGGL(score_kernel<5>, grid, block, 0, stream, a, b, d, rows_prev, n_prev, eps, scores, status);
  }
  if (n_win <= kWinThreads) {
    hipLaunchKernelGGL(window_topk_kernel<true>, dim3(unsigned(n_win)), dim3(kWinThreads), 0, stream, scores,
                       rows_prev, n_prev, T, window, pct, n_win, offs, n_out, rows_out, slot, status);
  } else {
    hipLaunchKernelGGL(window_count_kernel, dim3(1), dim3(kCountThreads), 0, stream, rows_prev, n_prev, T, window,
                       pct, n_win, n_out, offs, status);
    hipLaunchKernelGGL(window_topk_kernel<false>, dim3(unsigned(n_win)), dim3(kWinThreads), 0, stream, scores,
                       rows_prev, n_prev, T, window, pct, n_win, offs, n_out, rows_out, slot, status);
  }
  return hipGetLastError();
}

hipError_t launch_partition_rows(const uint8_t* cls, int32_t n, int32_t* gather, int32_t* scatter, int32_t* counts,
                                 uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(partition_kernel, dim3(1), dim3(kPartThreads), 0, stream, cls, n, gather, scatter, counts, status);
  return hipGetLastError();
}

}  // namespace flk
