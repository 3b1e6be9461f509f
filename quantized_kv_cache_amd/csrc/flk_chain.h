// flk_chain.h -- device-side reader of a packed loop chain for one 64-token x 128-channel tile.
//
// Used by the reconstruct kernel and the fused decode-attention kernel.  A 256-thread block
// covers the tile as 16 chunks of 8 channels (cc = tid & 15) times 16 row slots
// (rs = tid >> 4), each thread owning tokens t0 + rs + 16*i, i = 0..3.  Every element walks
// base -> delta2 -> ... in loop order, adding in binary32 and rounding to BF16 after each
// step exactly as the encoder did; a position a compact loop does not list inherits
// (FlashLoop RFC, vllm-rlt #156, section 3.3).
#pragma once

#include "flk_device.h"
#include "flk_internal.h"

namespace flk {

__device__ __forceinline__ int32_t lower_bound_rows(const int32_t* __restrict__ rows, int32_t n,
                                                    int32_t key) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    if (rows[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// lower_bound over an ascending array, computed by a whole 256-thread block in
// ceil(log256(n)) rounds of one parallel probe each (instead of log2(n) dependent loads):
// each round probes 256 evenly spaced entries of the current bracket and keeps the one
// stride that contains the first entry >= key.  Every thread returns the same value.
// Contains __syncthreads_count(); call from all threads of the block.
__device__ __forceinline__ int32_t block_lower_bound(const int32_t* __restrict__ rows, int32_t n,
                                                     int32_t key) {
  int32_t a = 0, b = n;                    // the answer lies in [a, b]
  while (a < b) {
    const int32_t s = (b - a + 255) / 256;
    const int32_t idx = a + int32_t(threadIdx.x) * s;
    const bool pred = idx < b && rows[idx] < key;
    const int32_t c = __syncthreads_count(pred);
    if (c == 0) return a;
    const int32_t na = a + (c - 1) * s + 1;
    const int32_t nb = min(a + c * s, b);
    if (s == 1) return nb;
    a = na;
    b = nb;
  }
  return a;
}

// lower_bound of `key` in every compact loop of a chain at once (dense loops give 0): the
// probes of all loops share each round, so the block waits ceil(log256(n)) load latencies
// in total rather than per loop.  Uniform control flow; call from all threads.
template <int NL>
__device__ __forceinline__ void chain_lower_bounds(const ChainArgs& chain, int32_t key,
                                                   int32_t lo[NL]) {
  int32_t a[NL], b[NL];
  bool done[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    a[l] = 0;
    b[l] = chain.s[l].rows ? chain.s[l].n : 0;
    done[l] = chain.s[l].rows == nullptr || b[l] == 0;
    lo[l] = 0;
  }
  for (int round = 0; round < 4; ++round) {
    bool any = false;
#pragma unroll
    for (int l = 0; l < NL; ++l) any |= !done[l];
    if (!any) break;
    bool pred[NL];
    int32_t st[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      st[l] = (b[l] - a[l] + 255) / 256;
      const int32_t idx = a[l] + int32_t(threadIdx.x) * st[l];
      pred[l] = !done[l] && idx < b[l] && chain.s[l].rows[idx] < key;
    }
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (done[l]) continue;
      const int32_t c = __syncthreads_count(pred[l]);
      if (c == 0) { lo[l] = a[l]; done[l] = true; continue; }
      const int32_t na = a[l] + (c - 1) * st[l] + 1;
      const int32_t nb = min(a[l] + c * st[l], b[l]);
      if (st[l] == 1 || na >= nb) { lo[l] = nb; done[l] = true; continue; }
      a[l] = na;
      b[l] = nb;
    }
  }
}

// lower_bound of key0 and of key1 in every compact loop of a chain (dense loops give 0),
// all probes sharing each round: ceil(log256(n)) load latencies in total.
template <int NL>
__device__ __forceinline__ void chain_bounds(const ChainArgs& chain, int32_t key0, int32_t key1,
                                             int32_t lo[NL], int32_t hi[NL]) {
  int32_t a[2][NL], b[2][NL];
  bool done[2][NL];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      a[k][l] = 0;
      b[k][l] = chain.s[l].rows ? chain.s[l].n : 0;
      done[k][l] = chain.s[l].rows == nullptr || b[k][l] == 0;
      (k ? hi : lo)[l] = 0;
    }
  for (int round = 0; round < 4; ++round) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int l = 0; l < NL; ++l) any |= !done[k][l];
    if (!any) break;
    bool pred[2][NL];
    int32_t st[2][NL];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        st[k][l] = (b[k][l] - a[k][l] + 255) / 256;
        const int32_t idx = a[k][l] + int32_t(threadIdx.x) * st[k][l];
        pred[k][l] = !done[k][l] && idx < b[k][l] && chain.s[l].rows[idx] < (k ? key1 : key0);
      }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        if (done[k][l]) continue;
        int32_t* res = k ? hi : lo;
        const int32_t c = __syncthreads_count(pred[k][l]);
        if (c == 0) { res[l] = a[k][l]; done[k][l] = true; continue; }
        const int32_t na = a[k][l] + (c - 1) * st[k][l] + 1;
        const int32_t nb = min(a[k][l] + c * st[k][l], b[k][l]);
        if (st[k][l] == 1 || na >= nb) { res[l] = nb; done[k][l] = true; continue; }
        a[k][l] = na;
        b[k][l] = nb;
      }
  }
}

// lower_bound of `key` in every compact loop of a chain, computed by one wave alone (no
// block barrier): each round probes 64 evenly spaced entries of every open bracket and keeps
// the stride holding the first entry >= key, so a loop of n rows needs ceil(log64(n)) rounds
// and all loops share them.  Returns wave-uniform values; dense loops give 0.
template <int NL>
__device__ __forceinline__ void wave_chain_lower_bounds(const ChainArgs& chain, int32_t key,
                                                        int32_t lo[NL]) {
  const int lane = threadIdx.x & 63;
  int32_t a[NL], b[NL];
  bool done[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    a[l] = 0;
    b[l] = chain.s[l].rows ? chain.s[l].n : 0;
    done[l] = chain.s[l].rows == nullptr || b[l] == 0;
    lo[l] = 0;
  }
  for (int round = 0; round < 6; ++round) {
    bool any = false;
#pragma unroll
    for (int l = 0; l < NL; ++l) any |= !done[l];
    if (!any) break;
    bool pred[NL];
    int32_t st[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      st[l] = (b[l] - a[l] + 63) / 64;
      const int32_t idx = a[l] + lane * st[l];
      pred[l] = !done[l] && idx < b[l] && chain.s[l].rows[idx] < key;
    }
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (done[l]) continue;
      const int32_t c = __builtin_popcountll(__ballot(pred[l]));
      if (c == 0) { lo[l] = a[l]; done[l] = true; continue; }
      const int32_t na = a[l] + (c - 1) * st[l] + 1;
      const int32_t nb = min(a[l] + c * st[l], b[l]);
      if (st[l] == 1 || na >= nb) { lo[l] = nb; done[l] = true; continue; }
      a[l] = na;
      b[l] = nb;
    }
  }
#pragma unroll
  for (int l = 0; l < NL; ++l) lo[l] = uniform(lo[l]);
}

// Fill s_map[l][i] with the compact row of position t0 + i in loop l (-1 if absent), for
// every compact loop of the chain.  Contains two __syncthreads(); call from all threads.
__device__ __forceinline__ void build_tile_maps(const ChainArgs& chain, int32_t t0,
                                                int32_t (*s_map)[kGroup]) {
  const int tid = threadIdx.x;
  const int n_loops = chain.n_loops;
  for (int idx = tid; idx < n_loops * kGroup; idx += blockDim.x) s_map[idx / kGroup][idx % kGroup] = -1;
  __syncthreads();
  for (int l = 1; l < n_loops; ++l) {
    const int32_t* rows = chain.s[l].rows;
    if (rows == nullptr) continue;
    const int32_t n = chain.s[l].n;
    const int32_t lo = lower_bound_rows(rows, n, t0);
    if (tid < kGroup) {
      const int32_t j = lo + tid;
      if (j < n) {
        const int32_t p = rows[j];
        if (p >= t0 && p < t0 + kGroup) s_map[l][p - t0] = j;
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void unpack_params8(const uint32_t* __restrict__ p, float m[8], float s[8]) {
  const uint4* pp = reinterpret_cast<const uint4*>(p);
  const uint4 a = pp[0], b = pp[1];
  const uint32_t pw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) { m[e] = f16_bits_to_f32(pw[e] & 0xFFFFu); s[e] = f16_bits_to_f32(pw[e] >> 16); }
}

// acc[i][e] = X_hat[R] at token t0 + rs + 16*i, channel ch + e (flattened H*D axis), as
// binary32 values that are exactly BF16.  tact[i] marks tokens inside [0, T).
template <int KIND>
__device__ __forceinline__ void read_chain_tile(const ChainArgs& chain, int32_t tile, int32_t T,
                                                int32_t H, int32_t D, int64_t ch, int rs,
                                                const int32_t (*s_map)[kGroup], float acc[4][8],
                                                bool tact[4]) {
  const int32_t t0 = tile * kGroup;
  const int32_t W = H * D;
  const int32_t S = (D + kGroup - 1) / kGroup;
  const int32_t h = int32_t(ch / D);
  const int32_t gsel = int32_t((ch - int64_t(h) * D) / kGroup);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tact[i] = (t0 + rs + 16 * i) < T;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
  }
  const int n_loops = chain.n_loops;
  for (int l = 0; l < n_loops; ++l) {
    const StreamArgs st = chain.s[l];
    const bool dense = st.rows == nullptr;
    float km[8], ks[8];
    if (KIND == FLK_KIND_K && dense) unpack_params8(st.params + int64_t(tile) * W + ch, km, ks);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!tact[i]) continue;
      const int32_t t = t0 + rs + 16 * i;
      const int32_t j = dense ? t : s_map[l][t - t0];
      if (j < 0) continue;
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(st.codes + ((int64_t(j) * W + ch) >> 1));
      float m[8], s[8];
      if (KIND == FLK_KIND_K) {
        if (dense) {
#pragma unroll
          for (int e = 0; e < 8; ++e) { m[e] = km[e]; s[e] = ks[e]; }
        } else {
          unpack_params8(st.params + int64_t(j / kGroup) * W + ch, m, s);
        }
      } else {
        const uint32_t pw = st.params[(int64_t(j) * H + h) * S + gsel];
        const float mm = f16_bits_to_f32(pw & 0xFFFFu), ss = f16_bits_to_f32(pw >> 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) { m[e] = mm; s[e] = ss; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = round_bf16(decode(nib(cw, e), m[e], s[e]));
        acc[i][e] = (l == 0) ? d : round_bf16(acc[i][e] + d);
      }
    }
  }
}

}  // namespace flk
