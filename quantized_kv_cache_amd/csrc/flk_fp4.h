// flk_fp4.h -- launchers of the FP4 (NVFP4, MXFP4) codec kernels, shared between the C-ABI
// front end and those kernels.
#pragma once

#include "flk_internal.h"

namespace flk {

// One FP4 stream of n rows of H*D channels: codes, block scales and the reconstruction
// (resid: against recon at rows, or at 0..n-1 when rows is NULL; compact loops also write
// tile_start).  NVFP4 (D % 16 == 0) first takes the stream amax into the params header (params:
// 16-byte header, then the E4M3 block scales); MXFP4 (mx, D % 32 == 0) writes the E8M0 block
// scales only.
hipError_t launch_fp4_encode(bool resid, bool mx, const void* x, const int32_t* rows, int32_t n, int32_t T,
                             int32_t H, int32_t D, void* recon, uint8_t* codes, uint32_t* params,
                             int32_t* tile_start, uint32_t* status, hipStream_t stream);

// X_hat [T, H, D] from a chain whose base (s[0]) is FP4 (base_fp4) or INT4 of the given kind and
// whose other loops are FP4; every FP4 loop is MXFP4 (mx) or every one NVFP4.
hipError_t launch_fp4_reconstruct(const ChainArgs& chain, bool base_fp4, bool mx, int kind, int32_t T, int32_t H,
                                  int32_t D, void* out, hipStream_t stream);

}  // namespace flk
