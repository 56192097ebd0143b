// Kernel entry points of the MFMA tiles; the tile body is in prefill_tile.h.
#include "prefill_tile.h"

namespace rpkv {

template <bool BIGPAGE>
__global__ __launch_bounds__(256, 2) void attn_prefill_bf16_kernel(AttnArgs a) {
  prefill_tile<BIGPAGE>(a, blockIdx.x);
}

int launch_prefill_bf16(const AttnArgs &a, void *stream) {
  if (a.n_items <= 0) return 0;
  // pages of >= 16 keys: a wavefront's 16 rows of a step share one page (steps
  // start on multiples of 64 keys: tiles start at key 0, cascade chunks at
  // multiples of 64)
  if (a.log2P >= 4)
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<true>, dim3(a.n_items), dim3(256), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(attn_prefill_bf16_kernel<false>, dim3(a.n_items), dim3(256), 0,
                       (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace rpkv
