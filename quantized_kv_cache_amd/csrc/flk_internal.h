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
  int32_t ktile;              // K parameter rows per 64-position tile (else per 64 compact rows)
};

// One encode of one tensor as a kernel sees it (single and batched calls alike).
struct EncArgs {
  const uint16_t* x;       // input rows [n][H][D]
  const int32_t* rows;     // compact positions (compact loops only)
  uint16_t* recon;         // X_hat [T][H][D]
  uint8_t* codes;
  uint32_t* params;
  int32_t* tile_start;     // compact loops only
  uint32_t* status;        // optional device status word
  int32_t n, T, W;         // rows, positions, channels per row (H*D)
  int32_t pos0;            // first position of the window (rows hold absolute positions)
  int32_t row0;            // rows of the stream before the window (offsets tile_start values)
  int32_t ktile;           // K groups per 64-position tile instead of per 64 compact rows
};

// Largest number of tensors one batched launch covers (the unit table travels as kernel
// arguments, at most 4 KiB; 56 covers every layer's K and V of a 24-layer request).
constexpr int kEncBatch = 56;

// Encode one loop (base when resid == false); a.rows == nullptr is a dense loop.  The
// pointers are already offset to the window (codes, params, tile_start).
hipError_t launch_encode(int kind, bool resid, const EncArgs& a, int32_t H, int32_t D, hipStream_t stream);

// p[0 .. count) = value (small fills of tile index entries and empty-tile parameters).
hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, hipStream_t stream);

// Whether a tensor of this kind and shape can join a batched encode launch; the others are
// encoded one launch each.
bool encode_batchable(int kind, int32_t H, int32_t D);

// The same loop type for n_units tensors, K and V mixed (kinds[i]), in launches of up to
// kEncBatch tensors.  Every tensor must be encode_batchable.
hipError_t launch_encode_batch(bool resid, bool sparse, const EncArgs* args, const int* kinds, int n_units,
                               hipStream_t stream);

hipError_t launch_reconstruct(int kind, int32_t T, int32_t H, int32_t D, const ChainArgs& chain,
                              void* out, hipStream_t stream);

// One reconstruct of a batched call.
struct RecArgs {
  ChainArgs chain;
  void* out;
  int32_t T, H, D, kind;
};
constexpr int kRecBatch = 8;

// Whether a tensor of this shape can join a batched reconstruct launch.
bool reconstruct_batchable(int32_t H, int32_t D);

// Rebuild n_units tensors (all reconstruct_batchable), K and V mixed: each run of consecutive
// units whose chains share loop count and compact pattern goes in launches of up to kRecBatch.
hipError_t launch_reconstruct_batch(const RecArgs* units, int n_units, hipStream_t stream);

}  // namespace flk
