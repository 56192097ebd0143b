// Kernel entry points of the MFMA tiles; the tile body is in prefill_tile.h.
#include "prefill_tile.h"

namespace rpkv {

template <int PM>
__global__ __launch_bounds__(256, 2) void attn_prefill_bf16_kernel(AttnArgs a) {
  prefill_tile<PM>(a, blockIdx.x);
}

int launch_prefill_bf16(const AttnArgs &a, void *stream) {
  if (a.n_items <= 0) return 0;
  // pages of >= 16 keys: a wavefront's 16 K rows of a step share one page;
  // pages of >= 4 keys: a lane's 4 V keys share one (steps start on multiples
  // of 64 keys: tiles at key 0, key splits and cascade chunks at multiples of 64)
  const dim3 grid(a.n_items), block(256);
  if (a.log2P >= 4)
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<2>, grid, block, 0, (hipStream_t)stream, a);
  else if (a.log2P >= 2)
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<1>, grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<0>, grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace rpkv
