// flk_select.h -- launchers of the token-selection and row-partition kernels, shared between
// the C-ABI front end and those kernels.
#pragma once

#include "flk_internal.h"

namespace flk {

int32_t select_windows(int32_t T, int32_t window);
size_t select_workspace_bytes(int32_t T, int32_t window);

// Scores (when 0 < pct < 100), window budgets, per-window top-k; arguments as flk_select_rows
// (validated by the caller).  hipErrorInvalidValue without launching for a short workspace or
// an unsupported d.
hipError_t launch_select_rows(const void* h_prev, const void* h_prev2, int32_t T, int32_t d, const int32_t* rows_prev,
                              int32_t n_prev, int32_t window, int32_t pct, float eps, float* scores,
                              int32_t* rows_out, int32_t n_out, int32_t* slot, void* ws, size_t ws_bytes,
                              uint32_t* status, hipStream_t stream);

hipError_t launch_partition_rows(const uint8_t* cls, int32_t n, int32_t* gather, int32_t* scatter, int32_t* counts,
                                 uint32_t* status, hipStream_t stream);

}  // namespace flk
