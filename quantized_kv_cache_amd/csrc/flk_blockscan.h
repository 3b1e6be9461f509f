// flk_blockscan.h -- block-wide scans shared by the top-k selections (sparse decode attention,
// token selection).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flk {

// Exclusive prefix of v over the NT threads of the block, and the total.  tmp holds NT/64
// entries.  Contains two __syncthreads(); call from all threads.
template <int NT>
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t* tmp, int32_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int32_t before = 0;
  total = 0;
  for (int u = 0; u < NT / 64; ++u) {
    before += u < wave ? tmp[u] : 0;
    total += tmp[u];
  }
  __syncthreads();
  return before + inc - v;
}

// The radix digit that holds the need-th largest key, from a histogram of nb <= 2 * NT digit
// counts: thread t owns digits nb-1-2t and nb-2-2t (counted from the top), a block scan gives
// the keys above each thread's pair, and the thread whose pair holds the need-th key writes
// the digit and the count of keys above it.  1 <= need <= the histogram's total.  Contains
// __syncthreads(); call from all threads.
template <int NT>
__device__ __forceinline__ void block_find_digit(const uint32_t* hist, uint32_t nb, uint32_t need, int32_t* tmp,
                                                 uint32_t& digit, uint32_t& above, uint32_t* s_digit,
                                                 uint32_t* s_above) {
  const int t = threadIdx.x;
  const int32_t d_hi = int32_t(nb) - 1 - 2 * t, d_lo = d_hi - 1;
  const uint32_t c_hi = d_hi >= 0 ? hist[d_hi] : 0u;
  const uint32_t c_lo = d_lo >= 0 ? hist[d_lo] : 0u;
  int32_t total;
  const uint32_t before = uint32_t(block_excl_scan<NT>(int32_t(c_hi + c_lo), tmp, total));
  if (before < need && need <= before + c_hi + c_lo) {
    if (before + c_hi >= need) {
      *s_digit = uint32_t(d_hi);
      *s_above = before;
    } else {
      *s_digit = uint32_t(d_lo);
      *s_above = before + c_hi;
    }
  }
  __syncthreads();
  digit = *s_digit;
  above = *s_above;
}

}  // namespace flk
