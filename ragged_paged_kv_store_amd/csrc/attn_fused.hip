// One launch for a mixed batch: the first blocks of the grid run split-KV
// chunks (4 wavefronts, one chunk each), the remaining blocks run MFMA tiles.
// Both kinds fit two workgroups per CU, so the chunks stream K/V from HBM on
// CUs beside the compute-bound tiles instead of waiting for them to finish
// (a mixed batch is split by token between decode and prefill work: SGLang
// source walkthrough "Attention backends", section 6).
#include "decode_chunk.h"
#include "prefill_tile.h"

namespace rpkv {

template <int PM>
__global__ __launch_bounds__(256, 2) void attn_fused_bf16_kernel(AttnArgs pre, AttnArgs dec,
                                                                 int32_t n_dec_blocks) {
  if ((int32_t)blockIdx.x < n_dec_blocks) {
    if (PM == 2)
      decode_chunk<dchunk::SlotsBig>(dec, blockIdx.x);
    else
      decode_chunk<dchunk::SlotsSmall>(dec, blockIdx.x);
    return;
  }
  prefill_tile<PM>(pre, blockIdx.x - n_dec_blocks);
}

int launch_fused_bf16(const AttnArgs &pre, const AttnArgs &dec, void *stream) {
  if (pre.n_items <= 0 && dec.n_items <= 0) return 0;
  // decode blocks padded to a multiple of the XCD count, so tile b of the
  // prefill list keeps running on XCD b % 8 as the planner arranged
  int32_t nd = (dec.n_items + kDecodeWavesPerBlock - 1) / kDecodeWavesPerBlock;
  nd = (nd + kNumXcd - 1) / kNumXcd * kNumXcd;
  const dim3 grid(nd + pre.n_items);
  const dim3 block(256);
  if (pre.log2P >= 4)
    hipLaunchKernelGGL(attn_fused_bf16_kernel<2>, grid, block, 0, (hipStream_t)stream, pre, dec, nd);
  else if (pre.log2P >= 2)
    hipLaunchKernelGGL(attn_fused_bf16_kernel<1>, grid, block, 0, (hipStream_t)stream, pre, dec, nd);
  else
    hipLaunchKernelGGL(attn_fused_bf16_kernel<0>, grid, block, 0, (hipStream_t)stream, pre, dec, nd);
  return (int)hipGetLastError();
}

}  // namespace rpkv
