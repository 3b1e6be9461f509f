// flk_internal.h -- launchers shared between the C-ABI front end and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/flk.h"

namespace flk {

// One loop of the chain as the kernels see it.
struct StreamArgs {
  const int32_t* rows;        // nullptr = dense
  const uint8_t* codes;
  const uint32_t* params;
  const int32_t* tile_start;  // inverse map per 64 positions (compact loops only)
  int32_t n;                  // compact rows
};

struct ChainArgs {
  StreamArgs s[FLK_MAX_LOOPS];
  int32_t n_loops;
};

// Encode one loop (base when resid == false).  Returns a hipError_t.
hipError_t launch_encode(int kind, bool resid, const void* x, const int32_t* rows, int32_t n,
                         int32_t T, int32_t H, int32_t D, void* recon, uint8_t* codes,
                         uint32_t* params, int32_t* tile_start, uint32_t* status,
                         hipStream_t stream);

hipError_t launch_reconstruct(int kind, int32_t T, int32_t H, int32_t D, const ChainArgs& chain,
                              void* out, hipStream_t stream);

size_t attn_workspace_bytes(int32_t T, int32_t H, int32_t Hq);

hipError_t launch_decode_attn(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, float scale, void* out,
                              void* ws, hipStream_t stream);

}  // namespace flk
