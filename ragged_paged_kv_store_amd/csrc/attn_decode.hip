// Kernel entry points of the split-KV chunks; the chunk body is in decode_chunk.h.
#include "decode_chunk.h"

namespace rpkv {

template <class Slots>
__global__ __launch_bounds__(256, 2) void attn_decode_bf16_kernel(AttnArgs a) {
  decode_chunk<Slots>(a, blockIdx.x);
}

int launch_decode_bf16(const AttnArgs &a, void *stream) {
  if (a.n_items <= 0) return 0;
  const int blocks = (a.n_items + kDecodeWavesPerBlock - 1) / kDecodeWavesPerBlock;
  // pages of >= 16 keys: 16-key blocks of a step lie in one page (chunks start
  // on multiples of 32 keys or at a cascade prefix length, a multiple of the page)
  if (a.log2P >= 4)
    hipLaunchKernelGGL(attn_decode_bf16_kernel<dchunk::SlotsBig>, dim3(blocks),
                       dim3(64 * kDecodeWavesPerBlock), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(attn_decode_bf16_kernel<dchunk::SlotsSmall>, dim3(blocks),
                       dim3(64 * kDecodeWavesPerBlock), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace rpkv
