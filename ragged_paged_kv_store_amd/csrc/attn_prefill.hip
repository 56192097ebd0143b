// bf16 MFMA attention tiles for prefill-type work and cascade prefix tiles.
//
// One workgroup (4 wavefronts) owns one tile of up to 128 query rows of one KV
// head: 128/G tokens x the G query heads that share the KV head (token-major),
// so every K/V byte staged in LDS feeds G heads.  Each wavefront owns 32 rows.
//
// Per 64-key step:
//  * the workgroup gathers 64 keys through the page table (16 B per thread per
//    load, coalesced along each 256-byte row) into registers one step ahead,
//    then writes K to LDS as [key][channel] and V transposed as [channel][key]
//    (4 keys x 8 channels per thread, transposed in registers), so both MFMA
//    A operands below are 16-byte LDS reads;
//  * S^T = K Q^T with 32x32x16 MFMAs (A = K rows, B = the wavefront's Q rows held
//    in registers): each lane then holds 32 logits of a single query row, so the
//    row max and sum are in-lane plus one cross-half shuffle;
//  * bottom-right causal mask (key <= position of the row's token; "The
//    attention backend and a reference implementation", "Variable-length, paged
//    attention with prefixes") only on steps that cross the diagonal or the key
//    range end; online softmax in base 2 with scale*log2(e) folded in;
//  * O^T += V^T P^T with 32x32x16 MFMAs; P^T comes straight from the S^T
//    accumulators (the key order inside the LDS V rows matches the order the
//    accumulator registers hold).
// A tile writes its final output, or a partial (normalised fp32 O and base-2
// log-sum-exp) when its key range is one of several (cascade prefix chunks).
#include "device_common.h"

namespace rpkv {

namespace {
constexpr int D = 128;
constexpr int BN = kPrefillKeys;  // 64 keys per step
constexpr int KS = D + 8;         // K LDS row stride (bf16), padded
constexpr int VS = BN + 8;        // V^T LDS row stride (bf16), padded
}  // namespace

__global__ __launch_bounds__(256, 2) void attn_prefill_bf16_kernel(AttnArgs a) {
  // two K/V buffers: step t computes from buffer t%2 while step t+1 is staged
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VS];

  const Item it = a.items[blockIdx.x];
  if (it.ntok == 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  // Running reference max (scaled, base 2) and this lane's part of the row sum.
  // The reference moves only when the row max passes it by more than 8, so the
  // exponentials stay <= 2^8 and the O rescale is skipped on most steps.
  float mref = kNegInf, lrun = 0.f;
  const float c = a.scale_log2;

  // ---- loader roles
  const int32_t *ptrow = a.page_table + (int64_t)it.req * a.pt_stride;
  const int pmask = (1 << a.log2P) - 1;
  const int kkey = tid >> 2, kpart = tid & 3;  // K: key, 32-channel quarter
  const int vkg = tid & 15, vdch = tid >> 4;   // V: keys 4*vkg..+3, channels 8*vdch..+7
  const char *kpool = (const char *)a.kpool;
  const char *vpool = (const char *)a.vpool;
  const int kbeg = it.kbeg, kend = it.kend;
  const int nsteps = (kend - kbeg + BN - 1) / BN;
  u32x4 kreg[4], vreg[4];
  int32_t pk, pv[4];  // page ids of the loader's keys for the next gather (-1: none)

  auto fetch_ids = [&](int kt) {
    const int key = kt + kkey;
    pk = key < kend ? ptrow[key >> a.log2P] : -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kv = kt + 4 * vkg + j;
      pv[j] = kv < kend ? ptrow[kv >> a.log2P] : -1;
    }
  };
  auto row_off = [&](int32_t page, int key) -> int64_t {
    const int64_t slot = ((int64_t)clamp_page(page, a.num_pages) << a.log2P) + (key & pmask);
    return (slot * a.Hkv + it.kvh) * (D * 2);
  };
  auto gather = [&](int kt) {
    if (pk >= 0) {
      const char *src = kpool + row_off(pk, kt + kkey) + kpart * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) kreg[j] = *(const u32x4 *)(src + 16 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) kreg[j] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (pv[j] >= 0)
        vreg[j] = *(const u32x4 *)(vpool + row_off(pv[j], kt + 4 * vkg + j) + vdch * 16);
      else
        vreg[j] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  // V key order inside a 16-key group of an LDS row: keys 0-3, 8-11, 4-7, 12-15,
  // so lane half h reads keys {4h..4h+3, 8+4h..8+4h+3} as one 16-byte vector.
  const int vslot = (vkg >> 2) * 16 + (vkg & 1) * 8 + ((vkg >> 1) & 1) * 4;
  auto stage = [&](int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4 *)&Ks[b][kkey * KS + kpart * 32 + 8 * j] = kreg[j];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int w = cc >> 1;
      const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
      u32x2 t;
      t[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
      t[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
      *(u32x2 *)&Vt[b][(8 * vdch + cc) * VS + vslot] = t;
    }
  };

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
    const uint16_t *Vb = Vt[t & 1];

    // ---- S^T = K Q^T: lane holds keys kt + 32*kb + (i/4)*8 + 4*half + i%4 of row m
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 kf = as_bf16x8(*(const u32x4 *)&Kb[(kb * 32 + q32) * KS + 16 * st + 8 * half]);
        s[kb] = mfma32(kf, qf[st], s[kb]);
      }
    }

    // ---- online softmax, base 2, scale folded into one FMA per logit
    if ((kt + BN - 1 > amin) || (kt + BN > kend)) {
      const int lim = min(kend - 1, apos);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt + 32 * kb + (i >> 2) * 8 + 4 * half + (i & 3);
          s[kb][i] = key <= lim ? s[kb][i] : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[kb][i], s[kb][i + 1]));
    mx = fmaxf(mx, shfl_xor(mx, 32)) * c;
    const bool upd = mx > mref + 8.f;
    if (upd) {
      const float al = fast_exp2(mref - mx);  // 0 on the first update
      lrun *= al;
      mref = mx;
      // scale this lane's O rows; lanes without an update keep theirs
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

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 vf = as_bf16x8(
              *(const u32x4 *)&Vb[(32 * db + q32) * VS + kb * 32 + s2 * 16 + half * 8]);
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

int launch_prefill_bf16(const AttnArgs &a, void *stream) {
  if (a.n_items <= 0) return 0;
  hipLaunchKernelGGL(attn_prefill_bf16_kernel, dim3(a.n_items), dim3(256), 0, (hipStream_t)stream,
                     a);
  return (int)hipGetLastError();
}

}  // namespace rpkv
