// bf16 MFMA attention tiles for prefill-type work and cascade prefix tiles.
//
// One workgroup (4 wavefronts) owns one tile of up to 128 query rows of one KV
// head: 128/G tokens x the G query heads that share the KV head (token-major),
// so every K/V byte staged in LDS feeds G heads.  (Where G does not divide 128
// a tile may instead hold 128 consecutive (token, head) rows starting inside a
// token: the item's row offset.)  Each wavefront owns 32 rows.
//
// Per 64-key step:
//  * K and V rows of the next step are gathered through the page table straight
//    into LDS with gfx950's global-to-LDS loads (16 bytes per lane, each
//    instruction filling 1 KiB = 4 rows), issued between the MFMAs of the
//    current step: no registers, no LDS store instructions, and the address
//    unit sees the loads spread over the step rather than in one burst.  K and
//    V each have two buffers, so a step's loads have the whole step to land.
//    Rows are 256 bytes, unpadded; chunk c of row r is stored at c ^ swz(r)
//    (swz swaps the two 2-bit halves of r % 16), which keeps both the 16-byte
//    K reads and the transposing V reads free of bank conflicts (an earlier
//    permutation, 2*(r%8) ^ (r/8)%2, left every transposing read 2-way
//    conflicted: 1.35 conflict cycles per LDS instruction in the hardware
//    counters, 0.03 now).  Keys past the range end load
//    a row of zeros (V rows must be finite: their weights are zero).  When a
//    page holds >= 16 keys, the 16 rows a wavefront loads lie in one page, so
//    the page id is a wave-uniform load;
//  * S^T = K Q^T with 32x32x16 MFMAs (A = K rows from LDS, B = the wavefront's Q
//    rows held in registers): each lane then holds 32 logits of a single query
//    row, so the row max and sum are in-lane plus one cross-half shuffle;
//  * bottom-right causal mask (key <= position of the row's token; "The
//    attention backend and a reference implementation", "Variable-length, paged
//    attention with prefixes") only on steps that cross the diagonal or the key
//    range end; online softmax in base 2 with scale*log2(e) folded into one FMA;
//    the O rescale is skipped unless the running max grows by more than 2^8;
//  * O^T += V^T P^T with 32x32x16 MFMAs: the V^T operand comes from row-major V
//    through the transposing LDS read (ds_read_b64_tr_b16: in each group of 16
//    lanes, lane i receives element i%4 of the 8-byte pieces addressed by lanes
//    4j + i/4, j = 0..3), and P^T straight from the S^T accumulators; the key
//    order the transposed reads produce matches the order the accumulators hold.
// A tile writes its final output, or a partial (normalised fp32 O and base-2
// log-sum-exp) when its key range is one of several (key splits of long
// prefills, cascade prefix chunks).
#pragma once

#include "device_common.h"

namespace rpkv {

namespace ptile {
constexpr int D = 128;
constexpr int BN = kPrefillKeys;  // 64 keys per step
constexpr int ROWB = D * 2;       // bytes per K/V row in LDS
constexpr int BUFB = BN * ROWB;   // bytes per K or V buffer
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 16-byte chunk permutation of LDS row r: chunk c of the row is stored at
// c ^ swz(r).  swz swaps the two 2-bit halves of r % 16: a bijection on 0..15
// (16 rows read at one logical chunk hit 16 different chunks), and 4 rows
// 4a..4a+3 map an aligned group of 4 chunks to 4 different groups (the 32
// lanes of a transposing read, 4 rows x 4 chunks, cover all 64 banks)
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ v4i16 tr_read(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16 *)(__attribute__((address_space(3))) void *)p);
}
}  // namespace ptile

// source of the rows of keys past the range end
static __device__ __attribute__((aligned(256))) uint32_t kZeroRow[ptile::ROWB / 4];

// PM: page mode.  2: pages of >= 16 keys; 1 and 0: smaller pages.
template <int PM>
__device__ __forceinline__ void prefill_tile(const AttnArgs &a, int tile) {
  using namespace ptile;
  constexpr bool BIGPAGE = PM == 2;
  // four separate arrays, each addressed statically below, so the compiler can
  // tell that loads into one buffer never alias reads of another
  __shared__ __attribute__((aligned(1024))) unsigned char K0[BUFB], K1[BUFB];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[BUFB], V1[BUFB];

  const Item it = a.items[tile];
  if (it.ntok == 0) return;
  // the wavefront index is uniform; saying so keeps per-wave values (page ids,
  // LDS destinations of the loads) in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int q32 = lane & 31, half = lane >> 5;
  const int G = a.G;
  const int ntok = item_ntok(it);
  const int rows = item_rows(it, G, kPrefillRows);
  const bool casc = it.pos0 < 0;

  // ---- this lane's query row (column of S^T); mr: its row in the token run
  const int m = wave * 32 + q32;
  const bool rowv = m < rows;
  const int mr = m + item_row0(it);
  const int tl = rowv ? mr / G : ntok - 1;
  const int gg = rowv ? mr % G : 0;
  const int tok = casc ? a.toklist[it.tok0 + tl] : it.tok0 + tl;
  const int qh = it.kvh * G + gg;
  const int apos = casc ? INT32_MAX : it.pos0 + tl;
  const int amin = casc ? INT32_MAX : it.pos0;  // smallest position in the tile
  // partial index base of this row's token, requested now and first used by the
  // epilogue (so the epilogue does not wait on a load)
  const int32_t pbase = it.split >= 0 ? a.tok_pbase[tok] : 0;

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

  // ---- loads: wavefront w fills rows 16w..16w+15 of a buffer with 4
  // instructions of 4 rows; in instruction i lane l fills chunk l%16 of row
  // 16w + 4i + l/16.
  const int32_t *ptrow = a.page_table + (int64_t)it.req * a.pt_stride;
  const int pmask = (1 << a.log2P) - 1;
  const int drow = lane >> 4, dpos = lane & 15;
  const char *kpool = (const char *)a.kpool;
  const char *vpool = (const char *)a.vpool;
  const int64_t row_bytes = (int64_t)a.Hkv * (D * 2);
  const int64_t head_off = (int64_t)it.kvh * (D * 2);
  const int kbeg = it.kbeg, kend = it.kend;
  const int nsteps = (kend - kbeg + BN - 1) / BN;
  // page ids of the next loads, of an in-range key (the key is clamped to the
  // range end): one per wavefront for big pages, else one per lane and row.
  // They are plain vector loads, requested a step ahead and first read after
  // the wait that ends that step, so reading them never waits on the
  // outstanding K/V loads.
  int32_t pg;
  int32_t pgl[4];

  auto page_of = [&](int key) { return ptrow[min(key, kend - 1) >> a.log2P]; };
  auto fetch_ids = [&](int kt) {
    if (BIGPAGE) {
      pg = page_of(kt + 16 * wave);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pgl[i] = page_of(kt + 16 * wave + 4 * i + drow);
    }
  };
  // Source addresses of the 4 K and 4 V load instructions of one step: row
  // 16*wave + 4i + drow, chunk ch_i = dpos ^ swz(4i + drow).  Steps start at
  // multiples of 64 keys, so with pages of >= 16 keys the wavefront's 16 rows
  // are the slots ((kt + 16w) % P) + 4i + drow of one page: a scalar base per
  // step plus a per-lane offset fixed for the whole tile.
  int32_t lane_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    lane_off[i] = (4 * i + drow) * (int32_t)row_bytes + (int32_t)head_off + 16 * (dpos ^ swz(4 * i + drow));
  const int64_t page_bytes = row_bytes << a.log2P;
  const char *ksrc[4], *vsrc[4];
  auto step_sources = [&](int kt) {
    if (BIGPAGE) {
      const int32_t p = clamp_page(__builtin_amdgcn_readfirstlane(pg), a.num_pages);
      const int64_t base = p * page_bytes + (int64_t)((kt + 16 * wave) & pmask) * row_bytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ksrc[i] = kpool + base + lane_off[i];
        vsrc[i] = vpool + base + lane_off[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * i + drow;
        const int64_t slot = ((int64_t)clamp_page(pgl[i], a.num_pages) << a.log2P) + ((kt + r) & pmask);
        const int64_t off = slot * row_bytes + head_off + 16 * (dpos ^ swz(r));
        ksrc[i] = kpool + off;
        vsrc[i] = vpool + off;
      }
    }
    if (kt + BN > kend) {  // the range ends in this step: rows past it read zeros
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = kt + 16 * wave + 4 * i + drow < kend;
        const char *z = (const char *)kZeroRow + 16 * (dpos ^ swz(4 * i + drow));
        ksrc[i] = valid ? ksrc[i] : z;
        vsrc[i] = valid ? vsrc[i] : z;
      }
    }
  };
  auto load_rows = [&](const char *src, unsigned char *buf, int i) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)(buf + (16 * wave + 4 * i) * ROWB),
                                     16, 0, 0);
  };

  // K reads: lane (q32, half) reads row 32*kb + q32, logical chunk 2*st + half
  const int kx = swz(q32);
  // V transposed reads: in 16-lane group g, lane 4j+q reads row 4*half + j (+8)
  // (+16*s2 + 32*kb), logical chunk 2*(g%2) + 4*db + q/2, bytes 8*(q%2)..
  const int vg = lane >> 4, vj = (lane & 15) >> 2, vq = lane & 3;
  const int vrow = 4 * half + vj;
  const int vx = swz(vrow), vxh = swz(vrow + 8);
  const int vc0 = 2 * (vg & 1) + (vq >> 1);

  // ---- prologue: step 0 loaded, ids of step 1 requested
  fetch_ids(kbeg);
  step_sources(kbeg);
#pragma unroll
  for (int i = 0; i < 4; ++i) load_rows(ksrc[i], K0, i);
#pragma unroll
  for (int i = 0; i < 4; ++i) load_rows(vsrc[i], V0, i);
  if (nsteps > 1) fetch_ids(kbeg + BN);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // one step: compute from (Kb, Vb), load the next step into (Kn, Vn)
  auto step = [&](int t, const unsigned char *Kb, const unsigned char *Vb, unsigned char *Kn,
                  unsigned char *Vn) {
    const int kt = kbeg + t * BN;
    // the last step loads rows past the range (zeros) into the idle buffers
    step_sources(kt + BN);

    // ---- S^T = K Q^T: lane holds keys kt + 32*kb + (i/4)*8 + 4*half + i%4 of row m;
    // two accumulation chains (key blocks 0 and 1); the next step's loads go
    // out between the MFMAs
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    // K fragments read two 16-channel slices ahead of the MFMAs that use them
    bf16x8 kf[3][2];
    auto kread = [&](int st, bf16x8(&dst)[2]) {
      const int ch = (2 * st + half) ^ kx;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        dst[kb] = as_bf16x8(*(const u32x4 *)(Kb + (kb * 32 + q32) * ROWB + 16 * ch));
    };
    kread(0, kf[0]);
    kread(1, kf[1]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st + 2 < 8) kread(st + 2, kf[(st + 2) % 3]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kf[st % 3][kb], qf[st], s[kb]);
      if (st & 1) load_rows(ksrc[st >> 1], Kn, st >> 1);
    }
    // keep that order: reads two slices ahead of their MFMAs, the next step's
    // K loads between them (0x100: LDS reads, 0x8: MFMA, 0x20: memory reads)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      // each K read right after the MFMA that consumed the register it refills
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (st + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (st & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
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
    // one 3-input max per two logits, in two independent chains
    float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      mx0 = fmaxf(fmaxf(mx0, s[0][i]), s[0][i + 1]);
      mx1 = fmaxf(fmaxf(mx1, s[1][i]), s[1][i + 1]);
    }
    float mx = max_halves(fmaxf(mx0, mx1)) * c;
    if (mx > mref + 8.f) {
      const float al = fast_exp2(mref - mx);  // 0 on the first update
      lrun *= al;
      mref = mx;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = o[db] * al;
    }
    const float mu = mref == kNegInf ? 0.f : mref;
    // the row sum adds the bf16 weights the PV product uses, two per instruction
    // (v_dot2 against (1, 1): exact products, fp32 sums), reading each finished
    // P fragment (its bf16 pairs taken as shuffles of the vector: as bit-cast
    // 32-bit lanes the compiler has fed one lane to two dot products)
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float sum0 = 0.f, sum1 = 0.f;
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
          w[j] = pack_bf16x2(p0, p1);
        }
        pf[kb][s2] = as_bf16x8(w);
        asm volatile("" : "+v"(pf[kb][s2]));
        const bf16x8 pv = pf[kb][s2];
        sum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 0, 1), ones, sum0, false);
        sum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 2, 3), ones, sum1, false);
        sum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 4, 5), ones, sum0, false);
        sum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 6, 7), ones, sum1, false);
      }
    lrun += sum0 + sum1;

    // ---- O^T += V^T P^T (V^T through the transposing LDS read)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const unsigned char *rp = Vb + (vrow + 16 * s2 + 32 * kb) * ROWB + 8 * (vq & 1);
          const v4i16 lo = tr_read(rp + 16 * ((vc0 + 4 * db) ^ vx));
          const v4i16 hi = tr_read(rp + 8 * ROWB + 16 * ((vc0 + 4 * db) ^ vxh));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = mfma32(vf, pf[kb][s2], o[db]);
          if (db == 3) load_rows(vsrc[2 * kb + s2], Vn, 2 * kb + s2);
        }
    // transposing reads one 16-key block ahead: the two reads of the next
    // block's fragment db right after the MFMA that consumed this block's
    // fragment db; a V load after each block (0x100: LDS reads, 0x8: MFMA,
    // 0x20: memory reads)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (blk + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
    }

    // ---- page ids for the loads of the step after next (the loads above used
    // the current ones); then the next step's rows have landed (this
    // wavefront's), then all waves
    if (t + 2 < nsteps) fetch_ids(kt + 2 * BN);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int t = 0; t < nsteps; t += 2) {
    step(t, K0, V0, K1, V1);
    if (t + 1 < nsteps) step(t + 1, K1, V1, K0, V0);
  }

  // ---- epilogue: this lane holds channels 32*db + (i/4)*8 + 4*half + i%4 of row m
  float l = sum_halves(lrun);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (it.split < 0) {
    // The rows leave through LDS (the last step's wait and barrier freed the
    // buffers): wavefront w writes its 32 rows into buffer w, row stride padded
    // by 16 bytes against bank conflicts, then stores whole 256-byte rows, 16
    // lanes per row and four rows per instruction, instead of 16-byte pieces
    // of 32 rows per instruction.
    constexpr int SROW = ROWB + 16;
    unsigned char *stg = wave == 0 ? K0 : wave == 1 ? K1 : wave == 2 ? V0 : V1;
    if (rowv) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w;
          w[0] = pack_bf16x2(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv);
          w[1] = pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
          *(u32x2 *)(stg + q32 * SROW + 2 * (32 * db + 8 * g4 + 4 * half)) = w;
        }
    }
    // the global row of each of the wavefront's rows, from the lane holding it
    const int64_t grow = (int64_t)tok * a.Hq + qh;
    const int32_t glo = (int32_t)grow, ghi = (int32_t)(grow >> 32);
    const int c16 = lane & 15, rsub = lane >> 4;
    unsigned char *out = (unsigned char *)a.out;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + rsub;
      const int64_t gr = ((int64_t)__shfl(ghi, r, 64) << 32) | (uint32_t)__shfl(glo, r, 64);
      if (wave * 32 + r < rows) {
        const u32x4 v = *(const u32x4 *)(stg + r * SROW + 16 * c16);
        *(u32x4 *)(out + gr * (D * 2) + 16 * c16) = v;
      }
    }
  } else {
    if (!rowv) return;
    // (the load of pbase is first read here: opaque until now, so no wait for
    // it is placed in the prologue)
    int32_t pb = pbase;
    asm volatile("" : "+v"(pb));
    const int64_t pi = (int64_t)pb + it.split;
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
