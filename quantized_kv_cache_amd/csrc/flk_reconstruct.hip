// flk_reconstruct.hip -- gfx950 reconstruction of X_hat[R] from a packed loop chain.
//
// One pass over the logical tensor: a block owns a 64-token tile (blockIdx.x) of a
// 128-channel strip (blockIdx.y) of the flattened H*D axis, reads every loop's codes and
// params for it once, and writes each output element once with a 16-byte store.
#include "flk_chain.h"

namespace flk {

constexpr int kRThreads = 256;

template <int KIND>
__global__ __launch_bounds__(kRThreads) void reconstruct_kernel(ChainArgs chain, int32_t T,
                                                                 int32_t H, int32_t D,
                                                                 uint16_t* __restrict__ out) {
  __shared__ int32_t s_map[FLK_MAX_LOOPS][kGroup];
  const int tid = threadIdx.x;
  const int cc = tid & 15;
  const int rs = tid >> 4;
  const int32_t W = H * D;
  const int chunk = blockIdx.y * 16 + cc;
  const int64_t ch = int64_t(chunk) * 8;

  build_tile_maps(chain, int32_t(blockIdx.x) * kGroup, s_map);
  if (chunk >= (W >> 3)) return;

  float acc[4][8];
  bool tact[4];
  read_chain_tile<KIND>(chain, blockIdx.x, T, H, D, ch, rs, s_map, acc, tact);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!tact[i]) continue;
    const int64_t t = int64_t(blockIdx.x) * kGroup + rs + 16 * i;
    uint4 w;
    w.x = pack_bf16x2(acc[i][0], acc[i][1]);
    w.y = pack_bf16x2(acc[i][2], acc[i][3]);
    w.z = pack_bf16x2(acc[i][4], acc[i][5]);
    w.w = pack_bf16x2(acc[i][6], acc[i][7]);
    *reinterpret_cast<uint4*>(out + t * W + ch) = w;
  }
}

hipError_t launch_reconstruct(int kind, int32_t T, int32_t H, int32_t D, const ChainArgs& chain,
                              void* out, hipStream_t stream) {
  const int32_t W = H * D;
  const dim3 grid(unsigned((T + kGroup - 1) / kGroup), unsigned((W / 8 + 15) / 16));
  if (kind == FLK_KIND_K)
    hipLaunchKernelGGL(reconstruct_kernel<FLK_KIND_K>, grid, dim3(kRThreads), 0, stream, chain, T,
                       H, D, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(reconstruct_kernel<FLK_KIND_V>, grid, dim3(kRThreads), 0, stream, chain, T,
                       H, D, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace flk
