// One launch for a mixed batch: the first blocks of the grid run split-KV
// chunks (one chunk per wavefront), the remaining blocks run MFMA tiles, one
// tile per 4-wavefront workgroup (two workgroups per CU) or two tiles per
// 8-wavefront workgroup in ping-pong.  Either way a CU holds 8 wavefronts, so
// the chunks stream K/V from HBM on CUs beside the compute-bound tiles instead
// of waiting for them to finish (a mixed batch is split by token between decode
// and prefill work: SGLang source walkthrough "Attention backends", section 6).
#include "decode_chunk.h"
#include "prefill_pair.h"

namespace rpkv {

template <int PM, int TPB>
__global__ __launch_bounds__(256 * TPB, 2) void attn_fused_bf16_kernel(AttnArgs pre, AttnArgs dec,
                                                                       int32_t n_dec_blocks) {
  if ((int32_t)blockIdx.x < n_dec_blocks) {
    if (PM == 2)
      decode_chunk<dchunk::SlotsBig, 4 * TPB>(dec, blockIdx.x);
    else
      decode_chunk<dchunk::SlotsSmall, 4 * TPB>(dec, blockIdx.x);
    return;
  }
  if (TPB == 2)
    prefill_pair<PM>(pre, blockIdx.x - n_dec_blocks);
  else
    prefill_tile<PM>(pre, blockIdx.x - n_dec_blocks);
}

template <int TPB>
static void launch_fused(const AttnArgs &pre, const AttnArgs &dec, hipStream_t stream) {
  // decode blocks padded to a multiple of the XCD count, so tile block b of the
  // prefill list keeps running on XCD b % 8 as the planner arranged
  constexpr int waves = 4 * TPB;
  int32_t nd = (dec.n_items + waves - 1) / waves;
  nd = (nd + kNumXcd - 1) / kNumXcd * kNumXcd;
  const dim3 grid(nd + (pre.n_items + TPB - 1) / TPB), block(256 * TPB);
  if (pre.log2P >= 4)
    hipLaunchKernelGGL((attn_fused_bf16_kernel<2, TPB>), grid, block, 0, stream, pre, dec, nd);
  else if (pre.log2P >= 2)
    hipLaunchKernelGGL((attn_fused_bf16_kernel<1, TPB>), grid, block, 0, stream, pre, dec, nd);
  else
    hipLaunchKernelGGL((attn_fused_bf16_kernel<0, TPB>), grid, block, 0, stream, pre, dec, nd);
}

int launch_fused_bf16(const AttnArgs &pre, const AttnArgs &dec, int tiles_per_block, void *stream) {
  if (pre.n_items <= 0 && dec.n_items <= 0) return 0;
  if (tiles_per_block == 2)
    launch_fused<2>(pre, dec, (hipStream_t)stream);
  else
    launch_fused<1>(pre, dec, (hipStream_t)stream);
  return (int)hipGetLastError();
}

}  // namespace rpkv
