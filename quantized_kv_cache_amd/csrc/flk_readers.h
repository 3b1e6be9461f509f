// flk_readers.h -- launchers of the kernels that read packed chains for attention (dense decode
// attention, sparse decode attention), shared between the C-ABI front end and those kernels.
#pragma once

#include "flk_internal.h"

namespace flk {

// Workspace of an attention call: exactly what a call over T packed tokens and a tail of
// tail_len tokens uses, and a bound for every split of T_total tokens into the two.
size_t attn_workspace_need(int32_t T, int32_t tail_len, int32_t H, int32_t Hq);
size_t attn_workspace_bytes(int32_t T_total, int32_t H, int32_t Hq);

// Packed positions [0, T) (T may be 0) plus an optional BF16 tail of tail_len positions.
// Returns hipErrorInvalidValue without launching when ws_bytes is below the need.
hipError_t launch_decode_attn(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, const void* k_tail,
                              const void* v_tail, int32_t tail_len, float scale, void* out,
                              void* ws, size_t ws_bytes, hipStream_t stream);

// launch_decode_attn over packed positions only, with the library's per-device scratch array as
// the workspace (no allocation); hipErrorInvalidValue without launching when the call needs
// more than FLK_NOALLOC_SCRATCH_BYTES.
hipError_t launch_decode_attn_noalloc(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q, const ChainArgs& kc,
                                      const ChainArgs& vc, float scale, void* out, hipStream_t stream);

// Decode attention over packed chains whose streams are INT4 throughout (fmt 0), an INT4 base
// with NVFP4 residual loops (fmt 1), NVFP4 throughout (fmt 2), an INT4 base with MXFP4 residual
// loops (fmt 3) or MXFP4 throughout (fmt 4), K and V alike; no tail.
hipError_t launch_decode_attn_fmt(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                                  const ChainArgs& vc, float scale, void* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

// Full attention over the packed chains (no tail) that also writes every scaled score to
// scores [Hq][T], the FP32 output to o_ref [Hq][128] and the softmax (max, denominator) to
// ml [Hq][2]; out gets the BF16 output.
hipError_t launch_attn_reference(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                                 const ChainArgs& vc, float scale, void* out, float* o_ref, float* ml,
                                 float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

// Sparse decode attention: workspace, the reference loop (after launch_attn_reference's
// attention) and a later loop; fmt as launch_decode_attn_fmt's.
size_t sparse_workspace_bytes(int32_t T, int32_t H, int32_t Hq, int32_t k, int32_t n_loops);
hipError_t launch_sparse_reference(int fmt, int32_t T, int32_t H, int32_t Hq, int32_t k, const void* q,
                                   const ChainArgs& kc, const ChainArgs& vc, float scale, void* out, int32_t* sel,
                                   float* mass, float* o_ref, float* c_ref, void* ws, size_t ws_bytes,
                                   hipStream_t stream);
hipError_t launch_sparse_loop(int fmt, int32_t T, int32_t H, int32_t Hq, int32_t k, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, float scale, const int32_t* sel,
                              const float* mass, const float* o_ref, const float* c_ref, void* out, void* ws,
                              size_t ws_bytes, hipStream_t stream);

}  // namespace flk
