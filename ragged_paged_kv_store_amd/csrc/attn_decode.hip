// Kernel entry points of the split-KV chunks; the chunk body is in decode_chunk.h.
#include "decode_chunk.h"

namespace rpkv {

// The planned split-KV launch runs two wavefronts (two chunks) per workgroup,
// 32 KiB of LDS, up to four workgroups per CU: a slot is handed to the next
// workgroup as soon as its two chunks end.  (Measured against four per
// workgroup: C3's launch 759 -> 723 us, 1.6-5.6% faster on other decode-only
// batches; one per workgroup was slower than both.)
constexpr int kPlannedDecodeWaves = 2;

template <class Slots>
__global__ __launch_bounds__(64 * kPlannedDecodeWaves, 8 / kPlannedDecodeWaves) void attn_decode_bf16_kernel(AttnArgs a) {
  // K rows staged in LDS, two steps per wavefront
  __shared__ __attribute__((aligned(1024))) unsigned char stage[kPlannedDecodeWaves * dchunk::kStageBytes];
  decode_chunk<Slots, kPlannedDecodeWaves>(a, blockIdx.x, stage);
}

int launch_decode_bf16(const AttnArgs &a, void *stream) {
  if (a.n_items <= 0) return 0;
  const int blocks = (a.n_items + kPlannedDecodeWaves - 1) / kPlannedDecodeWaves;
  // pages of >= 16 keys: 16-key blocks of a step lie in one page (chunks start
  // on multiples of 32 keys or at a cascade prefix length, a multiple of the page)
  if (a.log2P >= 4)
    hipLaunchKernelGGL(attn_decode_bf16_kernel<dchunk::SlotsBig>, dim3(blocks),
                       dim3(64 * kPlannedDecodeWaves), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(attn_decode_bf16_kernel<dchunk::SlotsSmall>, dim3(blocks),
                       dim3(64 * kPlannedDecodeWaves), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// Graph-capturable split-KV decode over a uniform batch (every request has
// q_len new tokens, packed request after request): wavefront ii runs key chunk
// c of request i for KV head h, ii = ((maxc - 1 - c) * batch + i) * Hkv + h, over
// keys [c * chunk, min(L_i, (c + 1) * chunk)); a chunk past L_i exits.  Chunk-major
// order from the last chunk down: the chunks past most requests' lengths are
// dispatched first and exit at once, the shorter last chunks of the long requests
// follow, and the grid ends on full-length first chunks, so no stream of empty
// wavefronts trails the work (measured: 2% faster than first-chunk-first).  L_i
// comes from seq_lens on the device, so one captured launch serves any lengths in
// [q_len, max_seq] (max_seq <= maxc * chunk); a request whose length is outside
// that range is skipped (no key is read, its output rows are not written).
// Token t's partial c is row t * maxc + c.
template <class Slots>
__global__ __launch_bounds__(256, 2) void attn_graph_decode_bf16_kernel(AttnArgs a,
                                                                        const int32_t *seq_lens,
                                                                        int32_t q_len, int32_t chunk,
                                                                        int32_t maxc, int32_t max_seq,
                                                                        int32_t batch) {
  __shared__ __attribute__((aligned(1024))) unsigned char stage[kDecodeWavesPerBlock * dchunk::kStageBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ii = blockIdx.x * kDecodeWavesPerBlock + wave;
  if (ii >= batch * maxc * a.Hkv) return;
  const int h = ii % a.Hkv, i = (ii / a.Hkv) % batch, c = maxc - 1 - ii / (a.Hkv * batch);
  const int L = seq_lens[i];
  if (L < q_len || L > max_seq) return;
  const int nch = (L + chunk - 1) / chunk;  // <= maxc
  if (c >= nch) return;
  const Item it{i, h, i * q_len, q_len, L - q_len, c * chunk, min(L, (c + 1) * chunk), nch > 1 ? c : -1};
  decode_item<Slots, true>(a, it, stage + wave * dchunk::kStageBytes);
}

int launch_graph_decode_bf16(const AttnArgs &a, const int32_t *seq_lens, int32_t q_len,
                             int32_t chunk, int32_t maxc, int32_t max_seq, int32_t batch,
                             void *stream) {
  const int32_t n_items = batch * maxc * a.Hkv;
  if (n_items <= 0) return 0;
  const int blocks = (n_items + kDecodeWavesPerBlock - 1) / kDecodeWavesPerBlock;
  const dim3 grid(blocks), block(64 * kDecodeWavesPerBlock);
  if (a.log2P >= 4)
    hipLaunchKernelGGL(attn_graph_decode_bf16_kernel<dchunk::SlotsBig>, grid, block, 0,
                       (hipStream_t)stream, a, seq_lens, q_len, chunk, maxc, max_seq, batch);
  else
    hipLaunchKernelGGL(attn_graph_decode_bf16_kernel<dchunk::SlotsSmall>, grid, block, 0,
                       (hipStream_t)stream, a, seq_lens, q_len, chunk, maxc, max_seq, batch);
  return (int)hipGetLastError();
}

}  // namespace rpkv
