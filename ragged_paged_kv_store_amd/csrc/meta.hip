// Packed-batch metadata on the device: the batch builder of "Variable-length
// batching and one mixed forward pass" (its worked example builds positions,
// query_start_loc, seq_lens, slot_mapping and logits_indices with a host loop;
// its source-code notes describe engines building them vectorised).  Two
// stream-ordered kernels, no host synchronisation, no allocation.
#include "device_common.h"

namespace rpkv {

// One workgroup: running sums of n and of need_logits over the batch in tiles
// of 1024 requests (wavefront scans, then a scan of the 16 wavefront totals).
__global__ __launch_bounds__(1024) void meta_scan_kernel(int32_t B, const int32_t *__restrict__ nc,
                                                         const int32_t *__restrict__ n,
                                                         const uint8_t *__restrict__ need,
                                                         int32_t *__restrict__ qsl,
                                                         int32_t *__restrict__ seq,
                                                         int32_t *__restrict__ lg,
                                                         int32_t *__restrict__ counts) {
  __shared__ int32_t wsum_t[16], wsum_l[16];
  __shared__ int32_t carry[2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    carry[0] = 0;
    carry[1] = 0;
    qsl[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    const int i = base + tid;
    const int ni = i < B ? n[i] : 0;
    const int li = (i < B && (need == nullptr || need[i])) ? 1 : 0;
    int st = ni, sl = li;  // inclusive scans within the wavefront
    for (int off = 1; off < 64; off <<= 1) {
      const int yt = __shfl_up(st, off, 64), yl = __shfl_up(sl, off, 64);
      if (lane >= off) {
        st += yt;
        sl += yl;
      }
    }
    if (lane == 63) {
      wsum_t[w] = st;
      wsum_l[w] = sl;
    }
    __syncthreads();
    int pt = carry[0], pl = carry[1];
    for (int k = 0; k < w; ++k) {
      pt += wsum_t[k];
      pl += wsum_l[k];
    }
    const int incl_t = pt + st;       // tokens of requests 0..i
    const int excl_l = pl + sl - li;  // requests before i that need logits
    if (i < B) {
      qsl[i + 1] = incl_t;
      seq[i] = nc[i] + ni;
      if (li) lg[excl_l] = incl_t - 1;
    }
    __syncthreads();  // every thread has read carry[]
    if (tid == 1023) {
      carry[0] = incl_t;
      carry[1] = excl_l + li;
    }
    __syncthreads();
  }
  if (tid == 0) {
    counts[0] = carry[0];
    counts[1] = carry[1];
  }
}

// One workgroup per request: positions and slots of its new tokens.
__global__ __launch_bounds__(256) void meta_tokens_kernel(
    const int32_t *__restrict__ nc, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ tables, int64_t stride, int32_t cols, int32_t log2P,
    int64_t max_tokens, int32_t *__restrict__ positions, int32_t *__restrict__ slots) {
  const int i = blockIdx.x;
  const int t0 = qsl[i], t1 = qsl[i + 1], c = nc[i];
  const int32_t *row = tables + (int64_t)i * stride;
  const int pmask = (1 << log2P) - 1;
  for (int t = t0 + (int)threadIdx.x; t < t1 && t < max_tokens; t += blockDim.x) {
    const int p = c + (t - t0);
    positions[t] = p;
    const int col = p >> log2P;
    slots[t] = col < cols ? (row[col] << log2P) + (p & pmask) : -1;
  }
}

int launch_build_metadata(int32_t B, const int32_t *nc, const int32_t *n, const uint8_t *need,
                          const int32_t *tables, int64_t stride, int32_t cols, int32_t log2P,
                          int64_t max_tokens, int32_t *qsl, int32_t *seq, int32_t *positions,
                          int32_t *slots, int32_t *lg, int32_t *counts, void *stream) {
  const hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(meta_scan_kernel, dim3(1), dim3(1024), 0, s, B, nc, n, need, qsl, seq, lg,
                     counts);
  if (B > 0)
    hipLaunchKernelGGL(meta_tokens_kernel, dim3(B), dim3(256), 0, s, nc, qsl, tables, stride, cols,
                       log2P, max_tokens, positions, slots);
  return (int)hipGetLastError();
}

// FlashInfer-style page table to the dense table the kernels read: row i gets
// the page ids page_indices[indptr[i] .. indptr[i+1]) ("SGLang source
// walkthrough, Attention backends", section 3.2).
__global__ __launch_bounds__(256) void csr_to_dense_kernel(const int32_t *__restrict__ indptr,
                                                           const int32_t *__restrict__ indices,
                                                           int32_t *__restrict__ dense,
                                                           int64_t stride) {
  const int i = blockIdx.x;
  const int a = indptr[i], b = indptr[i + 1];
  int32_t *row = dense + (int64_t)i * stride;
  for (int j = a + (int)threadIdx.x; j < b; j += blockDim.x) row[j - a] = indices[j];
}

// A block table for blocks of `factor` kernel pages each, rewritten into kernel
// pages: out[i][j*factor + r] = table[i][j]*factor + r (vLLM "Attention backends":
// the attention group's rewrite into kernel blocks).
__global__ __launch_bounds__(256) void rewrite_blocks_kernel(const int32_t *__restrict__ table,
                                                             int64_t stride, int32_t cols,
                                                             int32_t factor,
                                                             int32_t *__restrict__ out,
                                                             int64_t out_stride) {
  const int i = blockIdx.x;
  const int32_t *row = table + (int64_t)i * stride;
  int32_t *orow = out + (int64_t)i * out_stride;
  const int n = cols * factor;
  for (int j = threadIdx.x; j < n; j += blockDim.x) orow[j] = row[j / factor] * factor + j % factor;
}

int launch_csr_to_dense(int32_t B, const int32_t *indptr, const int32_t *indices, int32_t *dense,
                        int64_t stride, void *stream) {
  if (B <= 0) return 0;
  hipLaunchKernelGGL(csr_to_dense_kernel, dim3(B), dim3(256), 0, (hipStream_t)stream, indptr,
                     indices, dense, stride);
  return (int)hipGetLastError();
}

int launch_rewrite_blocks(int32_t B, const int32_t *table, int64_t stride, int32_t cols,
                          int32_t factor, int32_t *out, int64_t out_stride, void *stream) {
  if (B <= 0 || cols <= 0) return 0;
  hipLaunchKernelGGL(rewrite_blocks_kernel, dim3(B), dim3(256), 0, (hipStream_t)stream, table,
                     stride, cols, factor, out, out_stride);
  return (int)hipGetLastError();
}

}  // namespace rpkv
