// bf16 MFMA attention tiles, two per workgroup in ping-pong.
//
// A workgroup of 8 wavefronts runs two independent tiles (items 2p and 2p+1 of
// the prefill list), one per group of 4 wavefronts; wavefronts w and w+4 share
// a SIMD.  Each tile's work per 64-key step splits into a matrix phase (the
// MFMAs of S(t) = K(t) Q^T and of O += P(t-1) V(t-1)) and a vector phase (the
// online softmax of S(t) and the issue of later K/V loads).  The two groups run
// these phases in opposite order, separated by workgroup barriers, so on every
// SIMD one wavefront issues MFMAs while its partner does the softmax.
//
// Tile layout, masking, softmax and operand formats are those of the 4-wavefront
// tile (prefill_tile.h); only the schedule differs:
//   round r, group 0:  G(r) | V(r)          group 1:  V(r-1) | G(r)
//   G(r): S(r) from K buffer r%2, then O += P(r-1) V(r-1) from V buffer
//         (r-1)%2 (S(r) is complete by the time the vector phase reads it)
//   V(r): loads of K(r+2) into K buffer r%2 and of V(r+1) into V buffer
//         (r+1)%2; softmax of S(r) into P(r); wait for the loads issued in
//         V(r-1), which G(r+1) reads; page ids of step r+3.
// A tile of T steps runs rounds 0..T (G(T) is the last PV product) and writes
// its output right after round T.
// A buffer is refilled only after the barrier that ends the phase reading it,
// and loads have two phases to land.  A group whose tile has fewer steps keeps
// taking part in the barriers.
#pragma once

#include <type_traits>

#include "prefill_tile.h"

namespace rpkv {

namespace ppair {
// s_waitcnt immediate for "vector memory count <= n", other counters untouched
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
}  // namespace ppair

template <int PM, int GRP>
__device__ __forceinline__ void pair_group(const AttnArgs &a, const Item &it, const int T,
                                           const int R, const int lw) {
  using namespace ptile;
  constexpr bool BIGPAGE = PM == 2;
  constexpr int NIDS = BIGPAGE ? 0 : 4;  // vector loads per page-id fetch
  // per-group buffers (each instantiation has its own), addressed statically
  __shared__ __attribute__((aligned(1024))) unsigned char K0[BUFB], K1[BUFB];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[BUFB], V1[BUFB];

  if (T == 0) {  // no tile: keep the barrier count of the partner group
    for (int i = 0; i < 2 * R + 3; ++i) __builtin_amdgcn_s_barrier();
    return;
  }
  const int lane = threadIdx.x & 63;
  const int q32 = lane & 31, half = lane >> 5;
  const int G = a.G;
  const int rows = it.ntok * G;
  const bool casc = it.pos0 < 0;

  const int m = lw * 32 + q32;
  const bool rowv = m < rows;
  const int tl = rowv ? m / G : it.ntok - 1;
  const int gg = rowv ? m % G : 0;
  const int tok = casc ? a.toklist[it.tok0 + tl] : it.tok0 + tl;
  const int qh = it.kvh * G + gg;
  const int apos = casc ? INT32_MAX : it.pos0 + tl;
  const int amin = casc ? INT32_MAX : it.pos0;
  const int32_t pbase = it.split >= 0 ? a.tok_pbase[tok] : 0;

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
  const int kbeg = it.kbeg, kend = it.kend;

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
  const int vx = swz(vrow);
  const int vc0 = 2 * (vg & 1) + (vq >> 1);

  f32x16 s[2];
  bf16x8 pf[2][2];
  // page ids by step parity: at the start of V(r), ids[r%2] holds step r+2's
  // (K load) and ids[(r+1)%2] step r+1's (V load), which is then refetched for
  // step r+3; no id is ever copied, so no copy waits on its load
  Ids ids[2];

  // ---- prologue: K(0), V(0), K(1) loaded, ids of step 2 requested
  {
    Ids i0;
    fetch_ids(i0, kbeg);
    fetch_ids(ids[1], kbeg + BN);  // clamped in range when the tile has one step
    issue(i0, 0, kpool, K0);
    issue(i0, 0, vpool, V0);
    if (T > 1) issue(ids[1], 1, kpool, K1);
    ids[0] = i0;  // (a valid page for the loads past a short tile's end)
    if (T > 2) fetch_ids(ids[0], kbeg + 2 * BN);
    // the Q row goes out beside the first K/V loads, and one wait covers them
    // all: past it the compiler sees no vector load of its own pending (it
    // cannot see the K/V loads, and would otherwise wait on them for Q)
    const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)tok * a.Hq + qh) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*(const u32x4 *)(qrow + 16 * s + 8 * half));
    __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(0));
  }
  __builtin_amdgcn_s_barrier();

  // ---- matrix phase of round r
  auto gphase = [&](int r, const unsigned char *Kb, const unsigned char *Vp) {
    if (r > T) return;
    if (r < T) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
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
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (st + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      // the products stay in this phase
      asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    }
    if (r >= 1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const unsigned char *rp = Vp + (vrow + 16 * s2 + 32 * kb) * ROWB + 8 * (vq & 1);
            const v4i16 lo = tr_read(rp + 16 * ((vc0 + 4 * db) ^ vx));
            const v4i16 hi = tr_read(rp + 8 * ROWB + 16 * ((vc0 + 4 * db) ^ vx ^ 1));
            const bf16x8 vf = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = mfma32(vf, pf[kb][s2], o[db]);
          }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
        if (blk + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
      }
    }
  };

  auto epilogue = [&]() {
    float l = sum_halves(lrun);
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
      const int64_t pi = (int64_t)pbase + it.split;
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
    if ((kt + BN - 1 > amin) || (kt + BN > kend)) {
      const int rel = min(kend - 1, apos) - kt - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = (32 * kb + (i >> 2) * 8 + (i & 3)) <= rel ? s[kb][i] : kNegInf;
    }
    hook(0);
    // one 3-input max per two logits, in two independent chains
    float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      mx0 = fmaxf(fmaxf(mx0, s[0][i]), s[0][i + 1]);
      mx1 = fmaxf(fmaxf(mx1, s[1][i]), s[1][i + 1]);
    }
    float mx = max_halves(fmaxf(mx0, mx1)) * c;
    if (mx > mref + 8.f) {
      const float al = fast_exp2(mref - mx);
      lrun *= al;
      mref = mx;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = o[db] * al;
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
          const bf16x2 pp = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
          float &acc = (j & 1) ? sum1 : sum0;
          acc = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc, false);
          w[j] = __builtin_bit_cast(uint32_t, pp);
        }
        pf[kb][s2] = as_bf16x8(w);
        // computed here, not sunk toward its use in the next matrix phase
        // (past the barrier)
        asm volatile("" : "+v"(pf[kb][s2]));
        if (2 * kb + s2 < 3) hook(2 * kb + s2 + 1);
      }
    lrun += sum0 + sum1;
  };

  // ---- vector phase of round r: Kn = K buffer r%2, Vn = V buffer (r+1)%2;
  // P = r%2 (the parity is static in the unrolled loop).  With big pages the 8
  // loads go out two at a time between parts of the softmax, so their issue
  // (the address unit takes a while per 1 KiB load, and four wavefronts issue
  // together) overlaps the exponentials; with small pages they go out first.
  auto vphase = [&](int r, auto P, unsigned char *Kn, unsigned char *Vn) {
    if (r < 0 || r >= T) return;
    const bool f_ids = r + 3 < T, f_k = r + 2 < T, f_v = r + 1 < T;
    if (BIGPAGE) {
      // big pages: all 8 loads always go out (past the tile's last step they
      // refill buffers nobody reads), two at a time between parts of the
      // softmax, each from a scalar base plus a 32-bit lane offset
      uint32_t ok[4], ov[4];
      const char *sbk = step_addr(ids[P.value], r + 2, kpool, ok);
      const char *sbv = step_addr(ids[1 - P.value], r + 1, vpool, ov);
      softmax(r, [&](int h) {
        // the scheduler keeps each pair of loads between the blocks of work
        // around it
        __builtin_amdgcn_sched_barrier(0);
        if (h < 2) {
          load_rows_s(sbk, ok[2 * h], Kn, 2 * h);
          load_rows_s(sbk, ok[2 * h + 1], Kn, 2 * h + 1);
        } else {
          load_rows_s(sbv, ov[2 * h - 4], Vn, 2 * h - 4);
          load_rows_s(sbv, ov[2 * h - 3], Vn, 2 * h - 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      if (f_k) issue(ids[P.value], r + 2, kpool, Kn);
      if (f_v) issue(ids[1 - P.value], r + 1, vpool, Vn);
      softmax(r, [](int) {});
    }

    // the loads issued in the previous vector phase (read by the next matrix
    // phase) have landed; this phase's may still be in flight.  (Nothing of
    // the softmax is moved past the wait.)
    __builtin_amdgcn_sched_barrier(0);
    if (BIGPAGE || f_k)
      __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(8));
    else if (f_v)
      __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(4));
    else
      __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(0));
    // ids of step r+3, first read at the start of V(r+1)
    if (f_ids) fetch_ids(ids[1 - P.value], kbeg + (r + 3) * BN);
  };

  // ---- rounds 0..T of this tile, two at a time so every buffer is a fixed
  // array; then the output (outside the loop: the loop body stays small), then
  // the barriers of the partner's remaining rounds
  for (int r = 0; r <= T; r += 2) {
    if (GRP == 0) {
      gphase(r, K0, V1);
      __builtin_amdgcn_s_barrier();
      vphase(r, std::integral_constant<int, 0>(), K0, V1);
      __builtin_amdgcn_s_barrier();
    } else {
      vphase(r - 1, std::integral_constant<int, 1>(), K1, V0);
      __builtin_amdgcn_s_barrier();
      gphase(r, K0, V1);
      __builtin_amdgcn_s_barrier();
    }
    if (r + 1 > T) break;
    if (GRP == 0) {
      gphase(r + 1, K1, V0);
      __builtin_amdgcn_s_barrier();
      vphase(r + 1, std::integral_constant<int, 1>(), K1, V0);
      __builtin_amdgcn_s_barrier();
    } else {
      vphase(r, std::integral_constant<int, 0>(), K0, V1);
      __builtin_amdgcn_s_barrier();
      gphase(r + 1, K1, V0);
      __builtin_amdgcn_s_barrier();
    }
  }
  __builtin_amdgcn_s_waitcnt(ppair::vmcnt_imm(0));  // no load may outlive the workgroup
  epilogue();
  for (int i = 0; i < 2 * (R - T); ++i) __builtin_amdgcn_s_barrier();
}

// One workgroup of 8 wavefronts: items 2*pair (wavefronts 0-3) and 2*pair+1
// (wavefronts 4-7) of the list.
template <int PM>
__device__ __forceinline__ void prefill_pair(const AttnArgs &a, int pair) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i0 = 2 * pair, i1 = 2 * pair + 1;
  const Item it0 = a.items[i0];
  Item it1 = it0;
  it1.ntok = 0;
  if (i1 < a.n_items) it1 = a.items[i1];
  auto steps = [](const Item &it) {
    return it.ntok ? (it.kend - it.kbeg + ptile::BN - 1) / ptile::BN : 0;
  };
  const int T0 = steps(it0), T1 = steps(it1);
  const int R = max(T0, T1);
  if (R == 0) return;
  if (wave < 4)
    pair_group<PM, 0>(a, it0, T0, R, wave);
  else
    pair_group<PM, 1>(a, it1, T1, R, wave - 4);
}

}  // namespace rpkv
