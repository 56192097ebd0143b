// Kernel entry points of the MFMA tiles; the tile bodies are in prefill_tile.h
// (one tile per 4-wavefront workgroup) and prefill_pair.h (two tiles per
// 8-wavefront workgroup, in ping-pong).
#include "prefill_pair.h"

namespace rpkv {

template <int PM, int TPB>
__global__ __launch_bounds__(256 * TPB, 2) void attn_prefill_bf16_kernel(AttnArgs a) {
  if (TPB == 2)
    prefill_pair<PM>(a, blockIdx.x);
  else
    prefill_tile<PM>(a, blockIdx.x);
}

template <int TPB>
static void launch_prefill(const AttnArgs &a, hipStream_t stream) {
  // pages of >= 16 keys: a wavefront's 16 K rows of a step share one page;
  // pages of >= 4 keys: a lane's 4 V keys share one (steps start on multiples
  // of 64 keys: tiles at key 0, key splits and cascade chunks at multiples of 64)
  const dim3 grid((a.n_items + TPB - 1) / TPB), block(256 * TPB);
  if (a.log2P >= 4)
    hipLaunchKernelGGL((attn_prefill_bf16_kernel<2, TPB>), grid, block, 0, stream, a);
  else if (a.log2P >= 2)
    hipLaunchKernelGGL((attn_prefill_bf16_kernel<1, TPB>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_prefill_bf16_kernel<0, TPB>), grid, block, 0, stream, a);
}

int launch_prefill_bf16(const AttnArgs &a, int tiles_per_block, void *stream) {
  if (a.n_items <= 0) return 0;
  if (tiles_per_block == 2)
    launch_prefill<2>(a, (hipStream_t)stream);
  else
    launch_prefill<1>(a, (hipStream_t)stream);
  return (int)hipGetLastError();
}

}  // namespace rpkv
