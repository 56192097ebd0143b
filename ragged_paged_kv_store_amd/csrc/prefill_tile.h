// bf16 MFMA attention tiles for prefill-type work and cascade prefix tiles.
//
// One workgroup (4 wavefronts) owns one tile of up to 128 query rows of one KV
// head: 128/G tokens x the G query heads that share the KV head (token-major),
// so every K/V byte staged in LDS feeds G heads.  Each wavefront owns 32 rows.
//
// Per 64-key step:
//  * the workgroup gathers 64 K rows and 64 V rows of its KV head through the
//    page table (each thread 64 contiguous bytes of one row of each) one step
//    ahead into registers, and stores both row-major in LDS (288-byte rows, two
//    buffers).  When a page holds >= 16 keys the 16 rows a wavefront loads lie in
//    one page, so the page id is a wave-uniform load and the row addresses are a
//    scalar base plus a fixed lane offset;
//  * S^T = K Q^T with 32x32x16 MFMAs (A = K rows from LDS, B = the wavefront's Q
//    rows held in registers): each lane then holds 32 logits of a single query
//    row, so the row max and sum are in-lane plus one cross-half shuffle;
//  * bottom-right causal mask (key <= position of the row's token; "The
//    attention backend and a reference implementation", "Variable-length, paged
//    attention with prefixes") only on steps that cross the diagonal or the key
//    range end; online softmax in base 2 with scale*log2(e) folded into one FMA;
//    the O rescale is skipped unless the running max grows by more than 2^8;
//  * O^T += V^T P^T with 32x32x16 MFMAs: the V^T operand comes from row-major V
//    through gfx950's transposing LDS read (ds_read_b64_tr_b16: in each group of
//    16 lanes, lane i receives element i%4 of the 8-byte chunks addressed by
//    lanes 4j + i/4, j = 0..3), and P^T straight from the S^T accumulators; the
//    key order the transposed reads produce matches the order the accumulators
//    hold.
// A tile writes its final output, or a partial (normalised fp32 O and base-2
// log-sum-exp) when its key range is one of several (cascade prefix chunks).
#pragma once

#include "device_common.h"

namespace rpkv {

namespace ptile {
constexpr int D = 128;
constexpr int BN = kPrefillKeys;  // 64 keys per step
#ifndef VPAD
#define VPAD 16
#endif
// LDS row strides (bf16).  K rows are read 16 lanes x 16 B per pass, one row
// per lane: 272 B (68 dwords = 4 mod 64) puts 16 consecutive rows on distinct
// banks.  V rows are read by the transposing read, 4 rows x 32 B per 16-lane
// group, which wants the row stride apart by a multiple of 8 dwords.
constexpr int RSK = D + 8;
constexpr int RSV = D + VPAD;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ v4i16 tr_read(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16 *)(__attribute__((address_space(3))) void *)p);
}
}  // namespace ptile

template <bool BIGPAGE>
__device__ __forceinline__ void prefill_tile(const AttnArgs &a, int tile) {
  using namespace ptile;
  // two K/V buffers: step t computes from buffer t%2 while step t+1 is staged
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * RSK];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * RSV];

  const Item it = a.items[tile];
  if (it.ntok == 0) return;
  // the wavefront index is uniform; saying so lets per-wave addresses (the page
  // ids below) be scalar loads that do not wait on the vector-load counter
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int q32 = lane & 31, half = lane >> 5;
  const int G = a.G;
  const int rows = it.ntok * G;
  const bool casc = it.pos0 < 0;

  // ---- this lane's query row (column of S^T)
  const int m = wave * 32 + q32;
  const bool rowv = m < rows;
  const int tl = rowv ? m / G : it.ntok - 1;
  const int gg = rowv ? m % G : 0;
  const int tok = casc ? a.toklist[it.tok0 + tl] : it.tok0 + tl;
  const int qh = it.kvh * G + gg;
  const int apos = casc ? INT32_MAX : it.pos0 + tl;
  const int amin = casc ? INT32_MAX : it.pos0;  // smallest position in the tile

  bf16x8 qf[8];
  {
    const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)tok * a.Hq + qh) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*(const u32x4 *)(qrow + 16 * s + 8 * half));
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float mref = kNegInf, lrun = 0.f;
  const float c = a.scale_log2;

  // ---- loader: row lr (wavefront w owns rows 16w..16w+15), 64-byte quarter part
  const int32_t *ptrow = a.page_table + (int64_t)it.req * a.pt_stride;
  const int pmask = (1 << a.log2P) - 1;
  const int lr = tid >> 2, part = tid & 3;
  const char *kpool = (const char *)a.kpool;
  const char *vpool = (const char *)a.vpool;
  const int kbeg = it.kbeg, kend = it.kend;
  const int nsteps = (kend - kbeg + BN - 1) / BN;
  u32x4 kreg[4], vreg[4];
  int32_t pg;  // page id for the next gather, -1 when none of the rows is valid

  auto fetch_ids = [&](int kt) {
    if (BIGPAGE) {
      const int k0 = kt + 16 * wave;
      pg = __builtin_amdgcn_readfirstlane(k0 < kend ? ptrow[k0 >> a.log2P] : -1);
    } else {
      const int key = kt + lr;
      pg = key < kend ? ptrow[key >> a.log2P] : -1;
    }
  };
  auto gather = [&](int kt) {
    const int key = kt + lr;
    if (pg >= 0 && key < kend) {
      const int64_t slot = ((int64_t)clamp_page(pg, a.num_pages) << a.log2P) + (key & pmask);
      const int64_t off = (slot * a.Hkv + it.kvh) * (D * 2) + part * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) kreg[j] = *(const u32x4 *)(kpool + off + 16 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) vreg[j] = *(const u32x4 *)(vpool + off + 16 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kreg[j] = u32x4{0u, 0u, 0u, 0u};
        vreg[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stage = [&](int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4 *)&Ks[b][lr * RSK + part * 32 + 8 * j] = kreg[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4 *)&Vs[b][lr * RSV + part * 32 + 8 * j] = vreg[j];
  };
  // transposed V read of this lane: in its 16-lane group g, lane 4j+q points at
  // key row 4*half + j (+ 8*r) and channels 16*(g%2) + 4q (+ 32*db)
  const int vg = lane >> 4, vj = (lane & 15) >> 2, vq = lane & 3;
  const int vbase = (4 * half + vj) * RSV + 16 * (vg & 1) + 4 * vq;

  // ---- prologue: step 0 staged, step 1 in registers, ids of step 2 requested
  fetch_ids(kbeg);
  gather(kbeg);
  stage(0);
  if (nsteps > 1) {
    fetch_ids(kbeg + BN);
    gather(kbeg + BN);
  }
  if (nsteps > 2) fetch_ids(kbeg + 2 * BN);
  __syncthreads();

  for (int t = 0; t < nsteps; ++t) {
    const int kt = kbeg + t * BN;
    const uint16_t *Kb = Ks[t & 1];
    const uint16_t *Vb = Vs[t & 1];

    // ---- S^T = K Q^T: lane holds keys kt + 32*kb + (i/4)*8 + 4*half + i%4 of row m;
    // two independent accumulation chains (key blocks 0 and 1) interleaved
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = as_bf16x8(*(const u32x4 *)&Kb[(kb * 32 + q32) * RSK + 16 * st + 8 * half]);
        s[kb] = mfma32(kf, qf[st], s[kb]);
      }

    // ---- online softmax, base 2
    if ((kt + BN - 1 > amin) || (kt + BN > kend)) {
      const int rel = min(kend - 1, apos) - kt - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = (32 * kb + (i >> 2) * 8 + (i & 3)) <= rel ? s[kb][i] : kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kb][i], s[kb][i + 1]));
    mx = fmaxf(mx, shfl_xor(mx, 32)) * c;
    if (mx > mref + 8.f) {
      const float al = fast_exp2(mref - mx);  // 0 on the first update
      lrun *= al;
      mref = mx;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = o[db] * al;
    }
    const float mu = mref == kNegInf ? 0.f : mref;
    float sum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * s2 + 2 * j], c, -mu));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * s2 + 2 * j + 1], c, -mu));
          sum += p0 + p1;
          w[j] = pack_bf16x2(p0, p1);
        }
        pf[kb][s2] = as_bf16x8(w);
      }
    lrun += sum;

    // ---- O^T += V^T P^T (V^T through the transposing LDS read)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint16_t *vp = Vb + vbase + (kb * 32 + s2 * 16) * RSV + 32 * db;
          const v4i16 lo = tr_read(vp);
          const v4i16 hi = tr_read(vp + 8 * RSV);
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = mfma32(vf, pf[kb][s2], o[db]);
        }

    // ---- pipeline: stage step t+1, gather step t+2, request ids of step t+3
    if (t + 1 < nsteps) stage((t + 1) & 1);
    if (t + 2 < nsteps) gather(kt + 2 * BN);
    if (t + 3 < nsteps) fetch_ids(kt + 3 * BN);
    __syncthreads();
  }

  // ---- epilogue: this lane holds channels 32*db + (i/4)*8 + 4*half + i%4 of row m
  float l = lrun + shfl_xor(lrun, 32);
  if (!rowv) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (it.split < 0) {
    uint16_t *orow = (uint16_t *)a.out + ((int64_t)tok * a.Hq + qh) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv);
        w[1] = pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
        *(u32x2 *)(orow + 32 * db + 8 * g4 + 4 * half) = w;
      }
  } else {
    const int64_t pi = (int64_t)a.tok_pbase[tok] + it.split;
    float *prow = a.o_part + (pi * a.Hq + qh) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = o[db][4 * g4 + j] * inv;
        *(f32x4 *)(prow + 32 * db + 8 * g4 + 4 * half) = w;
      }
    if (half == 0) a.lse_part[pi * a.Hq + qh] = l > 0.f ? mref + fast_log2(l) : kNegInf;
  }
}

}  // namespace rpkv
