// store_kv scatter, log-sum-exp merge, and the fp32 attention kernel.
#include "device_common.h"

namespace rpkv {

// ---------------------------------------------------------------- store_kv
// store_kv / do_kv_cache_update (mini-sglang "The interface": write this
// step's K/V first; vLLM "Attention backends", Step 2: a scatter by slot).
// One thread moves one 16-byte chunk of one token's K row and V row; chunks of
// a row are contiguous, so a wavefront writes whole rows.  Negative and
// out-of-range slots write nothing.
__global__ __launch_bounds__(256) void store_kv_kernel(const u32x4 *__restrict__ k,
                                                       const u32x4 *__restrict__ v,
                                                       const int32_t *__restrict__ slots,
                                                       int64_t total, int32_t chunks_per_row,
                                                       int64_t num_slots, u32x4 *__restrict__ kpool,
                                                       u32x4 *__restrict__ vpool) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t t = i / chunks_per_row;
  const int32_t c = (int32_t)(i - t * chunks_per_row);
  // the row loads do not wait for the slot: one memory round trip, then stores
  const int32_t s = slots[t];
  const u32x4 kk = k[i];
  const u32x4 vv = v[i];
  if (s < 0 || s >= num_slots) return;
  const int64_t dst = (int64_t)s * chunks_per_row + c;
  kpool[dst] = kk;
  vpool[dst] = vv;
}

int launch_store_kv(const void *k, const void *v, const int32_t *slots, int64_t T,
                    int64_t row_bytes, int64_t num_slots, void *kpool, void *vpool,
                    void *stream) {
  if (T <= 0) return 0;
  const int32_t cpr = (int32_t)(row_bytes / 16);
  const int64_t total = T * cpr;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(store_kv_kernel, dim3((uint32_t)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4 *)k, (const u32x4 *)v, slots, total, cpr, num_slots,
                     (u32x4 *)kpool, (u32x4 *)vpool);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------- merge
// Combine the partial results of one token over disjoint key ranges (split-KV
// chunks, cascade prefix chunks and tails): with per-partial log-sum-exp l_s
// (base 2, of scaled logits) and normalised output o_s,
//   out = sum_s 2^(l_s - M) o_s / sum_s 2^(l_s - M),  M = max_s l_s,
// which is the softmax over the union of the key sets (SGLang walkthrough 3.3).
// A partial with l_s = -inf carries no weight.  One wavefront per (token, head):
// lane s holds partial s's weight (64 partials per pass), each lane D/64
// channels; the partial rows are independent loads issued back to back.
// All of a (token, head)'s log-sum-exps and partial rows requested at once (one
// memory round trip after the merge record), then combined; for ns <= NF.
template <int D, int NF>
__device__ __forceinline__ void merge_all_at_once(int32_t pb, int32_t ns, int h, int lane,
                                                  int64_t ob, const float *__restrict__ o_part,
                                                  const float *__restrict__ lse_part,
                                                  void *__restrict__ out, int32_t Hq,
                                                  int32_t dtype) {
  constexpr int PER = D / 64;
  const float *op = o_part + ((int64_t)pb * Hq + h) * D + lane * PER;
  const int64_t stride = (int64_t)Hq * D;
  const float lv = lane < ns ? lse_part[(int64_t)(pb + lane) * Hq + h] : kNegInf;
  float v[NF][PER];
#pragma unroll
  for (int u = 0; u < NF; ++u)
#pragma unroll
    for (int j = 0; j < PER; ++j) v[u][j] = u < ns ? op[u * stride + j] : 0.f;
  float M = lv;
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  const float wl = M == kNegInf ? 0.f : fast_exp2(lv - M);  // 2^-inf = 0
  float W = 0.f, acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
#pragma unroll
  for (int u = 0; u < NF; ++u) {
    const float w = __shfl(wl, u, 64);
    W += w;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += w * v[u][j];
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  if (dtype == RPKV_F32) {
#pragma unroll
    for (int j = 0; j < PER; ++j) ((float *)out)[ob + j] = acc[j] * inv;
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) ((uint16_t *)out)[ob + j] = f32_to_bf16(acc[j] * inv);
  }
}

template <int D>
__device__ __forceinline__ void merge_one(int32_t tok, int32_t pb, int32_t ns,
                                          const float *__restrict__ o_part,
                                          const float *__restrict__ lse_part,
                                          void *__restrict__ out, int32_t Hq, int32_t dtype) {
  constexpr int PER = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  if (h >= Hq) return;
  const int64_t ob = ((int64_t)tok * Hq + h) * D + lane * PER;
  // the usual cases: everything requested at once
  if (ns <= 8) return merge_all_at_once<D, 8>(pb, ns, h, lane, ob, o_part, lse_part, out, Hq, dtype);
  if (ns <= 32)
    return merge_all_at_once<D, 32>(pb, ns, h, lane, ob, o_part, lse_part, out, Hq, dtype);
  float M = kNegInf;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) M = fmaxf(M, lse_part[(int64_t)(pb + s0 + lane) * Hq + h]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float W = 0.f;
  if (M != kNegInf) {
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int cnt = min(64, ns - s0);
      const float lv = lane < cnt ? lse_part[(int64_t)(pb + s0 + lane) * Hq + h] : kNegInf;
      const float wl = fast_exp2(lv - M);  // 2^-inf = 0
      W += wl;
      const float *op = o_part + ((int64_t)(pb + s0) * Hq + h) * D + lane * PER;
      const int64_t stride = (int64_t)Hq * D;
      int s = 0;
      for (; s + 4 <= cnt; s += 4) {
        float v[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < PER; ++j) v[u][j] = op[(s + u) * stride + j];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = __shfl(wl, s + u, 64);
#pragma unroll
          for (int j = 0; j < PER; ++j) acc[j] += w * v[u][j];
        }
      }
      for (; s < cnt; ++s) {
        const float w = __shfl(wl, s, 64);
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += w * op[s * stride + j];
      }
    }
    for (int off = 32; off > 0; off >>= 1) W += shfl_xor(W, off);
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  if (dtype == RPKV_F32) {
#pragma unroll
    for (int j = 0; j < PER; ++j) ((float *)out)[ob + j] = acc[j] * inv;
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) ((uint16_t *)out)[ob + j] = f32_to_bf16(acc[j] * inv);
  }
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const int32_t *__restrict__ merge,
                                                    const float *__restrict__ o_part,
                                                    const float *__restrict__ lse_part,
                                                    void *__restrict__ out, int32_t Hq,
                                                    int32_t dtype) {
  merge_one<D>(merge[blockIdx.x * 3 + 0], merge[blockIdx.x * 3 + 1], merge[blockIdx.x * 3 + 2],
               o_part, lse_part, out, Hq, dtype);
}

// The graph-decode merge: token t of a uniform batch has ceil(L_i / chunk) <=
// maxc partials at rows t * maxc + c (none to merge when there is one: the chunk
// wrote the output); requests with L_i outside [q_len, max_seq] were skipped.
template <int D>
__global__ __launch_bounds__(256) void graph_merge_kernel(const int32_t *__restrict__ seq_lens,
                                                          int32_t q_len, int32_t chunk, int32_t maxc,
                                                          int32_t max_seq,
                                                          const float *__restrict__ o_part,
                                                          const float *__restrict__ lse_part,
                                                          void *__restrict__ out, int32_t Hq,
                                                          int32_t dtype) {
  const int32_t tok = blockIdx.x;
  const int32_t L = seq_lens[tok / q_len];
  if (L < q_len || L > max_seq) return;
  const int32_t ns = (L + chunk - 1) / chunk;  // <= maxc
  if (ns <= 1) return;
  merge_one<D>(tok, tok * maxc, ns, o_part, lse_part, out, Hq, dtype);
}

int launch_graph_merge(const int32_t *seq_lens, int32_t q_len, int32_t chunk, int32_t maxc,
                       int32_t max_seq, int32_t T, const float *o_part, const float *lse_part, void *out,
                       int32_t Hq, int32_t D, int32_t dtype, void *stream) {
  if (T <= 0) return 0;
  const dim3 grid(T, (Hq + 3) / 4);
  if (D == 128)
    hipLaunchKernelGGL(graph_merge_kernel<128>, grid, dim3(256), 0, (hipStream_t)stream, seq_lens,
                       q_len, chunk, maxc, max_seq, o_part, lse_part, out, Hq, dtype);
  else
    hipLaunchKernelGGL(graph_merge_kernel<64>, grid, dim3(256), 0, (hipStream_t)stream, seq_lens,
                       q_len, chunk, maxc, max_seq, o_part, lse_part, out, Hq, dtype);
  return (int)hipGetLastError();
}

int launch_merge(const int32_t *merge, int32_t n_merge, const float *o_part,
                 const float *lse_part, void *out, int32_t Hq, int32_t D, int32_t dtype,
                 void *stream) {
  if (n_merge <= 0) return 0;
  const dim3 grid(n_merge, (Hq + 3) / 4);
  if (D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, (hipStream_t)stream, merge, o_part,
                       lse_part, out, Hq, dtype);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, (hipStream_t)stream, merge, o_part,
                       lse_part, out, Hq, dtype);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------ fp32 kernel
// fp32 attention (the pages' fp32 path exists because the vendor kernels are
// bf16/fp16 only): vector ALU, one workgroup per item of up to 16 query rows,
// keys staged 32 at a time in LDS, online softmax per row.  Handles every item
// kind the planner emits (tiles, split-KV chunks, cascade prefix tiles).
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs a) {
  constexpr int R = kF32Rows, KB = kF32Keys;
  __shared__ float Qs[R][D];
  __shared__ float Ks[KB][D + 1];
  __shared__ float Vs[KB][D];
  __shared__ float Ps[R][KB + 1];
  __shared__ float m_s[R], l_s[R], al_s[R];
  __shared__ int32_t tok_s[R], qh_s[R], apos_s[R];
  __shared__ int64_t slot_s[KB];

  const Item it = a.items[blockIdx.x];
  if (it.ntok == 0) return;
  const int tid = threadIdx.x;
  const int G = a.G;
  const int rows = it.ntok * G;
  const bool casc = it.pos0 < 0;
  if (tid < R) {
    const int r = tid < rows ? tid : 0;
    const int tl = r / G;
    tok_s[tid] = casc ? a.toklist[it.tok0 + tl] : it.tok0 + tl;
    qh_s[tid] = it.kvh * G + r % G;
    apos_s[tid] = casc ? INT32_MAX : it.pos0 + tl;
    m_s[tid] = kNegInf;
    l_s[tid] = 0.f;
  }
  __syncthreads();
  for (int i = tid; i < R * D; i += 128) {
    const int r = i / D, d = i % D;
    Qs[r][d] = r < rows ? ((const float *)a.q)[((int64_t)tok_s[r] * a.Hq + qh_s[r]) * D + d] : 0.f;
  }
  constexpr int OUTS = R * D / 128;  // outputs per thread: rows r0 + j*RSTEP at channel d
  constexpr int RSTEP = 128 / D;
  const int od = tid % D, or0 = tid / D;
  float o[OUTS];
#pragma unroll
  for (int j = 0; j < OUTS; ++j) o[j] = 0.f;
  const int32_t *ptrow = a.page_table + (int64_t)it.req * a.pt_stride;
  const int32_t pmask = (1 << a.log2P) - 1;
  for (int kt = it.kbeg; kt < it.kend; kt += KB) {
    __syncthreads();
    if (tid < KB) {
      const int key = kt + tid;
      int64_t sl = -1;
      if (key < it.kend)
        sl = (int64_t)clamp_page(ptrow[key >> a.log2P], a.num_pages) * (pmask + 1) + (key & pmask);
      slot_s[tid] = sl;
    }
    __syncthreads();
    for (int i = tid; i < KB * D; i += 128) {
      const int j = i / D, d = i % D;
      const int64_t sl = slot_s[j];
      // keys past the range read slot 0 (always in bounds) and are zeroed
      const int64_t off = ((sl >= 0 ? sl : 0) * a.Hkv + it.kvh) * D + d;
      const float kx = ((const float *)a.kpool)[off];
      const float vx = ((const float *)a.vpool)[off];
      Ks[j][d] = sl >= 0 ? kx : 0.f;
      Vs[j][d] = sl >= 0 ? vx : 0.f;
    }
    __syncthreads();
    for (int p = tid; p < R * KB; p += 128) {
      const int r = p / KB, j = p % KB;
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) dot += Qs[r][d] * Ks[j][d];
      const int key = kt + j;
      const bool vis = key < it.kend && key <= apos_s[r];
      Ps[r][j] = vis ? dot * a.scale_log2 : kNegInf;
    }
    __syncthreads();
    if (tid < R) {
      float mx = kNegInf;
      for (int j = 0; j < KB; ++j) mx = fmaxf(mx, Ps[tid][j]);
      const float mn = fmaxf(m_s[tid], mx);
      const float mu = mn == kNegInf ? 0.f : mn;
      const float al = fast_exp2(m_s[tid] - mu);
      float sum = 0.f;
      for (int j = 0; j < KB; ++j) {
        const float pj = fast_exp2(Ps[tid][j] - mu);
        Ps[tid][j] = pj;
        sum += pj;
      }
      l_s[tid] = l_s[tid] * al + sum;
      m_s[tid] = mn;
      al_s[tid] = al;
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < OUTS; ++jj) {
      const int r = or0 + jj * RSTEP;
      float acc = o[jj] * al_s[r];
      for (int j = 0; j < KB; ++j) acc += Ps[r][j] * Vs[j][od];
      o[jj] = acc;
    }
  }
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < OUTS; ++jj) {
    const int r = or0 + jj * RSTEP;
    if (r >= rows) continue;
    const float l = l_s[r];
    const float val = l > 0.f ? o[jj] / l : 0.f;
    if (it.split < 0) {
      ((float *)a.out)[((int64_t)tok_s[r] * a.Hq + qh_s[r]) * D + od] = val;
    } else {
      const int64_t pi = (int64_t)a.tok_pbase[tok_s[r]] + it.split;
      a.o_part[(pi * a.Hq + qh_s[r]) * D + od] = val;
      if (od == 0) a.lse_part[pi * a.Hq + qh_s[r]] = l > 0.f ? m_s[r] + fast_log2(l) : kNegInf;
    }
  }
}

int launch_attn_f32(const AttnArgs &a, void *stream) {
  if (a.n_items <= 0) return 0;
  if (a.D == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(a.n_items), dim3(128), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(a.n_items), dim3(128), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace rpkv
