// bf16 MFMA attention tiles, two per workgroup in ping-pong, sharing K/V.
//
// A workgroup of 8 wavefronts runs two tiles (items 2p and 2p+1 of the prefill
// list), one per group of 4 wavefronts (group 0 on wavefronts 4-7, group 1 on
// 0-3); wavefronts w and w+4 share a SIMD.  The
// two tiles are siblings: query rows of the same request and KV head over the
// same first key (adjacent row blocks of one causal chunk, or of one cascade
// level chunk), so one stream of K/V rows staged in LDS serves both; the planner
// pairs them (an unpaired tile gets an empty partner, whose group then only
// loads).  Each tile's work per 64-key step splits into a matrix phase (the
// MFMAs of S(t) = K(t) Q^T and of O += P(t-1) V(t-1)) and a vector phase (the
// online softmax of S(t) and the issue of later loads).  The two groups run
// these phases in opposite order, separated by workgroup barriers, so on every
// SIMD one wavefront issues MFMAs while its partner does the softmax.
//
// Tile layout, masking and operand formats are those of the 4-wavefront tile
// (prefill_tile.h), and so is the softmax except for its reference (the row max
// of the first step only; see prefill_pair below); the schedule differs.  With
// half-round h:
//   round r, group 0:  G(r) [h = 2r]   | V(r)   [h = 2r+1]
//            group 1:  V(r-1) [h = 2r] | G(r)   [h = 2r+1]
//   G(r): S(r) from K(r) and O += P(r-1) V(r-1), interleaved (two 16-channel
//         slices of S, then one 16-key block of PV, four times), so the
//         transposing V reads spread over the phase instead of following
//         the K reads; round 0 multiplies a zeroed V buffer by P = 0 and
//         round T's S is discarded, so every round runs the same code
//   V(r): softmax of S(r) into P(r); group 0 loads K(r+2), group 1 loads
//         V(r+2) (four 1 KiB loads per wavefront); then the wait for the loads
//         this group issued in its previous vector phase.
// Step t's K and V sit in buffer t%3 of three: K(t) is read in half-rounds
// 2t and 2t+1 and refilled (with K(t+3)) in 2t+3; V(t) is read in 2t+2 and
// 2t+3 and refilled in 2t+4; every load has two half-rounds to land, and the
// barrier after the wait that covers it publishes it to the other group.  Both
// groups run the steps of the union of their key ranges; a group whose own range
// ends earlier masks the keys past it.  A tile of T steps runs rounds 0..T (G(T)
// is the last PV product) and writes its output right after round T.
#pragma once

#include <type_traits>

#include "prefill_tile.h"

namespace rpkv {

namespace ppair {
// s_waitcnt immediate for "vector memory count <= n", other counters untouched
// (clear bits 8-11 as well to wait for LDS and scalar memory too)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
}  // namespace ppair

// One group's tile of a pair (group GRP, its wavefronts lw = 0..3).  EXACT =
// false: each row's softmax reference is its max over the first step; returns
// true, having written nothing, when the workgroup must run its tiles again
// with EXACT = true, the running max of every step (see prefill_pair).
template <int PM, int GRP, bool EXACT>
__device__ __forceinline__ bool pair_group(const AttnArgs &a, const Item &it, const int kbeg,
                                           const int kend_u, const int T, unsigned char *Kbuf,
                                           unsigned char *Vbuf, const int lw, int *redo) {
  using namespace ptile;
  constexpr bool BIGPAGE = PM == 2;
  const bool own = it.ntok > 0;  // false: this group only loads (no tile)
  const int lane = threadIdx.x & 63;
  const int q32 = lane & 31, half = lane >> 5;
  const int G = a.G;
  const int ntok = item_ntok(it);
  const int rows = item_rows(it, G, kPrefillRows);
  const bool casc = it.pos0 < 0;

  // mr: this lane's row in the item's token run
  const int m = lw * 32 + q32;
  const bool rowv = m < rows;
  const int mr = m + item_row0(it);
  // (a group without a tile reads no token data)
  const int tl = rowv ? mr / G : (own ? ntok - 1 : 0);
  const int gg = rowv ? mr % G : 0;
  const int tok = !own ? 0 : casc ? a.toklist[it.tok0 + tl] : it.tok0 + tl;
  const int qh = it.kvh * G + gg;
  const int apos = casc ? INT32_MAX : it.pos0 + tl;
  const int amin = casc ? INT32_MAX : it.pos0;
  const int32_t pbase = own && it.split >= 0 ? a.tok_pbase[tok] : 0;

  bf16x8 qf[8];  // this lane's Q row, loaded in the prologue

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float mref = kNegInf, lrun = 0.f;
  const float c = a.scale_log2;

  const int32_t *ptrow = a.page_table + (int64_t)it.req * a.pt_stride;
  const int pmask = (1 << a.log2P) - 1;
  const int drow = lane >> 4, dpos = lane & 15;
  const char *kpool = (const char *)a.kpool;
  const char *vpool = (const char *)a.vpool;
  const int64_t row_bytes = (int64_t)a.Hkv * (D * 2);
  const int64_t head_off = (int64_t)it.kvh * (D * 2);
  // loads address the union of the two tiles' key ranges; the group's own end
  // masks its logits
  const int kend = kend_u, kend_own = it.kend;

  // page ids of one step's loads (see prefill_tile.h): one per wavefront for
  // big pages, a scalar load (the page table is constant during the launch;
  // scalar loads are counted apart from the K/V loads), else one per lane and
  // row
  struct Ids {
    int32_t pg;
    int32_t pgl[4];
  };
  const __attribute__((address_space(4))) int32_t *ptrow_c =
      (const __attribute__((address_space(4))) int32_t *)(uintptr_t)ptrow;
  auto page_of = [&](int key) { return ptrow[min(key, kend - 1) >> a.log2P]; };
  auto fetch_ids = [&](Ids &d, int kt) {
    if (BIGPAGE) {
      d.pg = ptrow_c[__builtin_amdgcn_readfirstlane(min(kt + 16 * lw, kend - 1) >> a.log2P)];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) d.pgl[i] = page_of(kt + 16 * lw + 4 * i + drow);
    }
  };
  int32_t lane_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    lane_off[i] = (4 * i + drow) * (int32_t)row_bytes + (int32_t)head_off + 16 * (dpos ^ swz(4 * i + drow));
  const int64_t page_bytes = row_bytes << a.log2P;
  // source rows of step `kt`'s loads into buffer rows 16*lw + 4i + drow
  auto sources = [&](const Ids &d, int kt, const char *pool, const char *(&src)[4]) {
    if (BIGPAGE) {
      const int32_t p = clamp_page(__builtin_amdgcn_readfirstlane(d.pg), a.num_pages);
      const int64_t base = p * page_bytes + (int64_t)((kt + 16 * lw) & pmask) * row_bytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) src[i] = pool + base + lane_off[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * lw + 4 * i + drow;
        const int64_t slot = ((int64_t)clamp_page(d.pgl[i], a.num_pages) << a.log2P) + ((kt + r) & pmask);
        src[i] = pool + slot * row_bytes + head_off + 16 * (dpos ^ swz(r));
      }
    }
    if (kt + BN > kend) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = kt + 16 * lw + 4 * i + drow < kend;
        src[i] = valid ? src[i] : (const char *)kZeroRow + 16 * (dpos ^ swz(4 * i + drow));
      }
    }
  };
  // The K/V loads are written as instructions the compiler does not track:
  // it would otherwise make later LDS reads (and reuse of address registers)
  // wait for every load in flight, including those into the other buffers.
  // The waits are explicit instead: each vector phase ends waiting for the
  // loads issued in the previous one, and a barrier follows.
  auto lds_addr = [&](unsigned char *buf, int i) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)(buf + (16 * lw + 4 * i) * ROWB);
  };
  auto load_rows = [&](const char *src, unsigned char *buf, int i) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_addr(buf, i)) : "memory");
  };
  auto load_rows_s = [&](const char *sbase, uint32_t off, unsigned char *buf, int i) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sbase), "{m0}"(lds_addr(buf, i))
                 : "memory");
  };
  // (big pages) scalar base of this wavefront's 16 rows of step t
  auto step_base = [&](const Ids &d, int t, const char *pool) {
    const int32_t p = clamp_page(__builtin_amdgcn_readfirstlane(d.pg), a.num_pages);
    return pool + (p * page_bytes + (int64_t)((kbeg + t * BN + 16 * lw) & pmask) * row_bytes);
  };
  // (big pages) base and lane offsets of this wavefront's 16 rows of step t.
  // Rows past the range end read the range's last row instead (finite data;
  // their logits are masked), and a block wholly past it reads the last
  // 16-key block: in-page offsets, so one scalar base serves all rows.
  const int lastblk = (kend - 1) & ~15;
  auto step_addr = [&](const Ids &d, int t, const char *pool, uint32_t (&off)[4]) {
    const int ebs = min(kbeg + t * BN + 16 * lw, lastblk);
    const int jmax = min(15, kend - 1 - ebs);
    const int32_t p = clamp_page(__builtin_amdgcn_readfirstlane(d.pg), a.num_pages);
    if (jmax == 15) {
#pragma unroll
      for (int i = 0; i < 4; ++i) off[i] = (uint32_t)lane_off[i];
    } else {
      // (a real branch: the clamped offsets are computed only on this path)
      asm volatile("");
#pragma unroll
      for (int i = 0; i < 4; ++i)
        off[i] = (uint32_t)(lane_off[i] + (min(4 * i + drow, jmax) - (4 * i + drow)) * (int32_t)row_bytes);
    }
    return pool + (p * page_bytes + (int64_t)(ebs & pmask) * row_bytes);
  };
  // Loads of step t into `buf`.  With big pages, steps before the range end
  // address a scalar base plus the fixed 32-bit lane offsets; otherwise per-lane
  // addresses, rows past the range end reading zeros.
  auto issue = [&](const Ids &d, int t, const char *pool, unsigned char *buf) {
    const int kt = kbeg + t * BN;
    if (BIGPAGE && kt + BN <= kend) {
      const char *sbase = step_base(d, t, pool);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_rows_s(sbase, (uint32_t)lane_off[i], buf, i);
      return;
    }
    const char *src[4];
    sources(d, kt, pool, src);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_rows(src[i], buf, i);
  };

  const int kx = swz(q32);
  const int vg = lane >> 4, vj = (lane & 15) >> 2, vq = lane & 3;
  const int vrow = 4 * half + vj;
  const int vx = swz(vrow), vxh = swz(vrow + 8);
  const int vc0 = 2 * (vg & 1) + (vq >> 1);

  f32x16 s[2];
  // P(r-1) of the PV product; zero before the first step (the first matrix
  // phase's PV then adds nothing)
  bf16x8 pf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[kb][s2][i] = (__bf16)0.f;
  // this group's share of the loads: K rows (group 0) or V rows (group 1) of
  // each step, rows 16*lw.. of the buffer of the step
  const char *pool = GRP == 0 ? kpool : vpool;
  unsigned char *const LB = GRP == 0 ? Kbuf : Vbuf;
  // page ids of the step the next vector phase loads (fetched at the end of the
  // vector phase before it; one slot, never copied)
  Ids ids;

  // ---- prologue: steps 0 and 1 of this group's share loaded, ids of step 2
  // requested
  {
    Ids i0, i1;
    fetch_ids(i0, kbeg);
    fetch_ids(i1, kbeg + BN);  // clamped in range when there is one step
    issue(i0, 0, pool, LB);
    issue(i1, 1, pool, LB + BUFB);
    fetch_ids(ids, kbeg + 2 * BN);
    // the Q row goes out beside the first loads, and one wait covers them
    // all: past it the compiler sees no vector load of its own pending (it
    // cannot see the K/V loads, and would otherwise wait on them for Q)
    if (own) {
      const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)tok * a.Hq + qh) * D;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*(const u32x4 *)(qrow + 16 * s + 8 * half));
    }
    // V(-1): buffer 2, read (with zero weights) in round 0, must hold finite
    // values: 8 wavefronts x 2 x 1 KiB of zeros
    {
      const int w8 = GRP == 0 ? 4 + lw : lw;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *(u32x4 *)(Vbuf + 2 * BUFB + (w8 * 2 + i) * 1024 + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
    }
    // (the zeros and every load have landed before the barrier)
    __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(0) & ~(15 << 8));
  }
  __builtin_amdgcn_s_barrier();

  // ---- matrix phase of round r
  // (B: r % 3, a compile-time constant in the unrolled loop below, so every
  // LDS address is a fixed offset)
  auto gphase = [&](int r, auto B) {
    if (!own || r > T) return;
    // the wavefront issuing MFMAs goes first when its SIMD partner (in its
    // vector phase) also has an instruction ready
    __builtin_amdgcn_s_setprio(3);
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char *Kb = Kbuf + B.value * BUFB;
    const unsigned char *Vp = Vbuf + ((B.value + 2) % 3) * BUFB;  // V(r-1)
    // S(r) = K(r) Q^T in four pairs of 16-channel slices, each followed by one
    // 16-key block of O += P(r-1) V(r-1): every 8 MFMAs carry 4 K reads and 8
    // transposing V reads, so LDS work is spread evenly over the phase.  (Round
    // 0 adds P = 0 times a zeroed V buffer; round T's S is not used.)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    auto kread = [&](int st, bf16x8(&dst)[2]) {
      const int ch = (2 * st + half) ^ kx;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        dst[kb] = as_bf16x8(*(const u32x4 *)(Kb + (kb * 32 + q32) * ROWB + 16 * ch));
    };
    auto vread = [&](int blk, bf16x8(&dst)[4]) {
      const int kb = blk >> 1, s2 = blk & 1;
      const unsigned char *rp = Vp + (vrow + 16 * s2 + 32 * kb) * ROWB + 8 * (vq & 1);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const v4i16 lo = tr_read(rp + 16 * ((vc0 + 4 * db) ^ vx));
        const v4i16 hi = tr_read(rp + 8 * ROWB + 16 * ((vc0 + 4 * db) ^ vxh));
        dst[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    bf16x8 kf[2][2], vf[4];
    kread(0, kf[0]);
    kread(1, kf[1]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      vread(u, vf);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kf[h][kb], qf[2 * u + h], s[kb]);
      if (u < 3) {
        // (written last-needed first: the scheduler places them in reverse)
        auto kread_rev = [&](int st, bf16x8(&dst)[2]) {
          const int ch = (2 * st + half) ^ kx;
#pragma unroll
          for (int kb = 1; kb >= 0; --kb)
            dst[kb] = as_bf16x8(*(const u32x4 *)(Kb + (kb * 32 + q32) * ROWB + 16 * ch));
        };
        kread_rev(2 * u + 3, kf[1]);
        kread_rev(2 * u + 2, kf[0]);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = mfma32(vf[db], pf[u >> 1][u & 1], o[db]);
    }
    // order: the first pair's K reads; then per unit, the S MFMAs with the
    // unit's V reads two after each, the PV MFMAs with the next pair's K reads
    // one after each (0x100: LDS reads, 0x8: MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (u < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // the products stay in this phase
    asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  // The output rows leave through LDS: each wavefront writes its 32 rows there
  // (row stride padded by 16 bytes against bank conflicts), then stores whole
  // 256-byte rows, 16 lanes per row and four rows per instruction.  (Stored
  // straight from the accumulators, every instruction wrote 16-byte pieces of
  // 32 rows, and a workgroup retires only once its stores are acknowledged:
  // C4's launch took 3% longer.)  The K/V buffers are free by then.
  auto epilogue = [&]() {
    float l = sum_halves(lrun);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (it.split < 0) {
      constexpr int SROW = ROWB + 16;
      unsigned char *stg = (GRP == 0 ? Kbuf : Vbuf) + lw * (32 * SROW);
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
        if (lw * 32 + r < rows) {
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
  };

  // softmax of S(r) into P(r); hook(h) runs before the row max (h = 0) and
  // after each of the first three 16-key blocks of exponentials (h = 1..3)
  auto softmax = [&](int r, auto &&hook) {
    const int kt = kbeg + r * BN;
    if ((kt + BN - 1 > amin) || (kt + BN > kend_own)) {
      const int rel = min(kend_own - 1, apos) - kt - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = (32 * kb + (i >> 2) * 8 + (i & 3)) <= rel ? s[kb][i] : kNegInf;
    }
    hook(0);
    if (EXACT || r == 0) {
      // one 3-input max per two logits, in two independent chains
      float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        mx0 = fmaxf(fmaxf(mx0, s[0][i]), s[0][i + 1]);
        mx1 = fmaxf(fmaxf(mx1, s[1][i]), s[1][i + 1]);
      }
      const float mx = max_halves(fmaxf(mx0, mx1)) * c;
      if (mx > mref + 8.f) {
        const float al = fast_exp2(mref - mx);
        lrun *= al;
        mref = mx;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = o[db] * al;
      }
    }
    const float mu = mref == kNegInf ? 0.f : mref;
    // the row sum adds the bf16 weights the PV product uses, two per
    // instruction (v_dot2 against (1, 1): exact products, fp32 sums)
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float sum0 = 0.f, sum1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * s2 + 2 * j], c, -mu));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * s2 + 2 * j + 1], c, -mu));
          w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
        }
        // computed here, not sunk toward its use in the next matrix phase
        // (past the barrier)
        pf[kb][s2] = as_bf16x8(w);
        asm volatile("" : "+v"(pf[kb][s2]));
        // the sums read the finished P registers, so the packed words need no
        // second home.  (Operands taken as shuffles of the bf16 vector: taken
        // as bit-cast 32-bit lanes of it, the compiler fed one lane to two
        // dot products.)
        {
          const bf16x8 pv = pf[kb][s2];
          sum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 0, 1), ones, sum0, false);
          sum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 2, 3), ones, sum1, false);
          sum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 4, 5), ones, sum0, false);
          sum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 6, 7), ones, sum1, false);
        }
        if (2 * kb + s2 < 3) hook(2 * kb + s2 + 1);
      }
    lrun += sum0 + sum1;
  };

  // ---- vector phase of round r: the group's four loads of step r+2 into
  // buffer (r+2)%3 (read last in half-round 2r-1 for K, 2r+1 for V), the
  // softmax of S(r), the wait for the loads of the previous vector phase, the
  // ids of step r+3.  With big pages the loads go out one between each part of
  // the softmax, from a scalar base plus 32-bit lane offsets (past the range
  // end they refill a buffer nobody reads); with small pages they go out first.
  auto vphase = [&](int r, auto B) {
    if (r < 0 || r >= T) return;
    unsigned char *dst = LB + ((B.value + 2) % 3) * BUFB;
    if (BIGPAGE) {
      uint32_t off[4];
      const char *sb = step_addr(ids, r + 2, pool, off);
      // the ids of step r+3 go out now (a scalar load: the next matrix
      // phase's first LDS wait would otherwise cover it too)
      fetch_ids(ids, kbeg + (r + 3) * BN);
      if (own) {
        softmax(r, [&](int h) {
          // the scheduler keeps each load between the blocks of work around it
          __builtin_amdgcn_sched_barrier(0);
          load_rows_s(sb, off[h], dst, h);
          __builtin_amdgcn_sched_barrier(0);
        });
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) load_rows_s(sb, off[i], dst, i);
      }
    } else {
      issue(ids, r + 2, pool, dst);
      if (own) softmax(r, [](int) {});
    }
    // the loads of the previous vector phase (read from the next half-round on)
    // have landed; this phase's may still be in flight.  (Nothing of the
    // softmax is moved past the wait.)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(4));
    if (!BIGPAGE) fetch_ids(ids, kbeg + (r + 3) * BN);
  };

  // ---- rounds 0..T, three at a time so every buffer is a fixed address; then
  // the output
  auto round = [&](int r, auto B) {
    if (GRP == 0) {
      gphase(r, B);
      __builtin_amdgcn_s_barrier();
      vphase(r, B);
      __builtin_amdgcn_s_barrier();
    } else {
      vphase(r - 1, std::integral_constant<int, (B.value + 2) % 3>());
      __builtin_amdgcn_s_barrier();
      gphase(r, B);
      __builtin_amdgcn_s_barrier();
    }
  };
  for (int r = 0; r <= T; r += 3) {
    round(r, std::integral_constant<int, 0>());
    if (r + 1 > T) break;
    round(r + 1, std::integral_constant<int, 1>());
    if (r + 2 > T) break;
    round(r + 2, std::integral_constant<int, 2>());
  }
  __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(0));  // no load may outlive the workgroup
  // every wavefront's loads have landed and its LDS reads are done (the fences
  // wait for them): the buffers may be written again
  __syncthreads();
  if (!EXACT) {
    // a weight sum at or above 2^64, inf or NaN asks for the second pass (bit
    // patterns of non-negative floats order as integers)
    if (own && __any(__builtin_bit_cast(uint32_t, lrun) >= 0x5f800000u) && lane == 0) *redo = 1;
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(*(volatile int *)redo) != 0) return true;
  }
  if (own) epilogue();
  return false;
}

// One workgroup of 8 wavefronts: items 2*pair (group 0, on wavefronts 4-7) and
// 2*pair+1 (group 1, on wavefronts 0-3) of the list, siblings sharing one K/V
// stream.  (Group 0 runs its matrix phase first; on the younger wavefronts it
// balances the two half-rounds better: an SIMD's older wavefront wins issue
// when both have an instruction ready.)  A unit whose first item is padding is
// skipped; an empty second item makes group 1 a loader for group 0's tile.
template <int PM>
__device__ __forceinline__ void prefill_pair(const AttnArgs &a, int pair) {
  using namespace ptile;
  __shared__ __attribute__((aligned(1024))) unsigned char Kbuf[3 * BUFB], Vbuf[3 * BUFB];
  __shared__ int redo;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i0 = 2 * pair, i1 = 2 * pair + 1;
  const Item it0 = a.items[i0];
  if (it0.ntok == 0) return;
  Item it1 = it0;
  it1.ntok = 0;
  if (i1 < a.n_items && a.items[i1].ntok > 0) it1 = a.items[i1];
  const int kend_u = max(it0.kend, it1.kend);
  const int T = (kend_u - it0.kbeg + BN - 1) / BN;
  if (threadIdx.x == 0) redo = 0;  // published by the groups' first barrier
  // First pass: each row's weights are taken against its max over the tile's
  // first step, and later steps take no row max at all (the softmax does not
  // depend on the reference; only the range of the weights does).  A weight
  // exceeds 1 where a later logit exceeds that max, and is at most the row's
  // weight sum; while every sum stays below 2^64 no weight, sum or output can
  // overflow (for values of V below 2^60).  Otherwise the workgroup runs its
  // tiles again with the running max of every step (second pass, EXACT).
  const bool again = wave >= 4 ? pair_group<PM, 0, false>(a, it0, it0.kbeg, kend_u, T, Kbuf, Vbuf, wave - 4, &redo)
                                : pair_group<PM, 1, false>(a, it1, it0.kbeg, kend_u, T, Kbuf, Vbuf, wave, &redo);
  if (again) {
    // the items read afresh (the values of the first pass are not kept for
    // this one), made uniform again field by field
    auto item_at = [&](int i) {
      const int32_t *src = (const int32_t *)(a.items + i);
      Item v;
      int32_t *dst = (int32_t *)&v;
#pragma unroll
      for (int f = 0; f < 8; ++f) dst[f] = __builtin_amdgcn_readfirstlane(((const volatile int32_t *)src)[f]);
      return v;
    };
    const Item r0 = item_at(i0);
    Item r1 = r0;
    r1.ntok = 0;
    if (i1 < a.n_items) {
      const Item t1 = item_at(i1);
      if (t1.ntok > 0) r1 = t1;
    }
    const int ke = max(r0.kend, r1.kend);
    const int Tr = (ke - r0.kbeg + BN - 1) / BN;
    if (wave >= 4)
      pair_group<PM, 0, true>(a, r0, r0.kbeg, ke, Tr, Kbuf, Vbuf, wave - 4, &redo);
    else
      pair_group<PM, 1, true>(a, r1, r0.kbeg, ke, Tr, Kbuf, Vbuf, wave, &redo);
  }
}

}  // namespace rpkv
