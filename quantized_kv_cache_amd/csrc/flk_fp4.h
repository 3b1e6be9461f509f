// flk_fp4.h -- launchers of the NVFP4 codec kernels, shared between the C-ABI front end and
// those kernels.
#pragma once

#include "flk_internal.h"

namespace flk {

// One NVFP4 stream of n rows of H*D channels (D % 16 == 0): the stream amax into the params
// header, then codes, block scales, header and the reconstruction (resid: against recon at
// rows, or at 0..n-1 when rows is NULL; compact loops also write tile_start).  params is the
// stream's params buffer (16-byte header, then the block scales).
hipError_t launch_fp4_encode(bool resid, const void* x, const int32_t* rows, int32_t n, int32_t T, int32_t H,
                             int32_t D, void* recon, uint8_t* codes, uint32_t* params, int32_t* tile_start,
                             uint32_t* status, hipStream_t stream);

// X_hat [T, H, D] from a chain whose base (s[0]) is NVFP4 (base_fp4) or INT4 of the given kind
// and whose other loops are NVFP4.
hipError_t launch_fp4_reconstruct(const ChainArgs& chain, bool base_fp4, int kind, int32_t T, int32_t H, int32_t D,
                                  void* out, hipStream_t stream);

}  // namespace flk
