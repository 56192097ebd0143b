// bf16 split-KV decode attention for gfx950.
//
// Decode-type work ("Variable-length batching and one mixed forward pass",
// exercise 2: pure decode uses split-KV / flash-decoding kernels) is bound by
// reading K and V from HBM.  One wavefront owns one item: up to 16 query rows
// (n tokens x G heads of one KV head, token-major) against a contiguous key
// chunk of one request.  Each K/V byte of the chunk is read from HBM once and
// serves all G heads.
//
// Per 32-key step the wavefront:
//  * gets K as MFMA A operands (lane = key, lane group = 8 channels of a
//    32-channel slice): in a launch of its own, staged through LDS by
//    global-to-LDS loads of whole 256-byte rows and read back with
//    ds_read_b128 (see load_k_lds); beside MFMA tiles, loaded straight into
//    registers (16 B per lane per load),
//  * computes S^T = K Q^T with 16x16x32 bf16 MFMAs (2 key blocks x 4 channel
//    slices); query columns beyond the item's rows are zero,
//  * applies the bottom-right mask (key <= position of the column's token) and
//    the chunk end, and updates the online softmax with wavefront shuffles
//    across the four lane groups that share a column,
//  * loads V rows (16 B per lane: 8 channels of one key), transposes them in
//    registers into A operands of O^T = V^T P^T, and accumulates with 8 MFMAs
//    (output row m of virtual block c is channel 8m + c).
// K and V are read with nontemporal loads: each byte is read once (a read-only
// probe streams 7.0 TB/s so, against 6.3-6.8 with plain loads; a batch of 256
// decodes over 1k-8k keys runs 6% faster).  Loads of step t+1 and page-table
// reads of step t+2 are issued before step t is computed (two register or
// LDS sets, no copies); page ids are scalar loads.
// The item writes its rows' final output, or a partial result (normalised O in
// fp32 plus the base-2 log-sum-exp) for the merge kernel.
#pragma once

#include "device_common.h"

namespace rpkv {

namespace dchunk {

constexpr int D = 128;

struct Regs {
  u32x4 k[2][4];
  u32x4 v[8];
};

// Keys of one 32-key step held by this lane:
//  K (A operand of S^T): key kb + 16*sb + col for sb = 0, 1
//  V (A operand of O^T): key kb + 16*(e/4) + 4*grp + e%4, e = 0..7
//
// Small pages (< 16 keys): every key's slot is looked up; keys at or past kend
// are clamped to kend - 1 (always readable) and masked.
struct SlotsSmall {
  int32_t k[2];
  int32_t v[8];
};
// Pages of >= 16 keys: steps start on multiples of 16 keys, so keys
// kb..kb+15 and kb+16..kb+31 each lie in one page; the two page ids are
// wave-uniform.  Keys past the range read in-page rows (their page index is
// clamped to the last page in range) and are masked; their V rows are zeroed.
struct SlotsBig {
  int32_t pg[2];
};

__device__ __forceinline__ int32_t slot_of(const int32_t *ptrow, int key, int kend, int log2P,
                                           int64_t num_pages) {
  const int kc = key < kend ? key : kend - 1;
  const int pg = clamp_page(ptrow[kc >> log2P], num_pages);
  return (pg << log2P) + (kc & ((1 << log2P) - 1));
}

// byte offset of channel 0 of KV head kvh in pool slot `slot`
__device__ __forceinline__ int64_t row_bytes_off(int32_t slot, int hkv, int kvh) {
  return ((int64_t)(uint32_t)slot * hkv + kvh) * (D * 2);
}

__device__ __forceinline__ void lookup(SlotsSmall &s, const int32_t *ptrow, int kb, int kend,
                                       int col, int grp, int log2P, int64_t num_pages) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) s.k[sb] = slot_of(ptrow, kb + 16 * sb + col, kend, log2P, num_pages);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = kb + (e >> 2) * 16 + 4 * grp + (e & 3);
    s.v[e] = slot_of(ptrow, key, kend, log2P, num_pages);
  }
}

__device__ __forceinline__ void lookup(SlotsBig &s, const int32_t *ptrow, int kb, int kend, int,
                                       int, int log2P, int64_t num_pages) {
  // scalar loads through the constant address space (the page table does not
  // change during the launch): counted apart from the K/V loads, so using the
  // ids never waits for K/V in flight
  const __attribute__((address_space(4))) int32_t *ptc =
      (const __attribute__((address_space(4))) int32_t *)(uintptr_t)ptrow;
  const int last = (kend - 1) >> log2P;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int pi = __builtin_amdgcn_readfirstlane(min((kb + 16 * sb) >> log2P, last));
    s.pg[sb] = __builtin_amdgcn_readfirstlane(clamp_page(ptc[pi], num_pages));
  }
}

__device__ __forceinline__ void load(Regs &r, const SlotsSmall &s, const char *kpool,
                                     const char *vpool, int, int col, int grp, int, int hkv,
                                     int kvh) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      r.k[sb][st] =
          __builtin_nontemporal_load((const u32x4 *)(kpool + row_bytes_off(s.k[sb], hkv, kvh) + (st * 32 + grp * 8) * 2));
#pragma unroll
  for (int e = 0; e < 8; ++e)
    r.v[e] = __builtin_nontemporal_load((const u32x4 *)(vpool + row_bytes_off(s.v[e], hkv, kvh) + col * 16));
}

__device__ __forceinline__ void load(Regs &r, const SlotsBig &s, const char *kpool,
                                     const char *vpool, int kb, int col, int grp, int log2P,
                                     int hkv, int kvh) {
  const int pmask = (1 << log2P) - 1;
  const int64_t rowb = (int64_t)hkv * (D * 2);  // bytes between consecutive slots
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    // first slot of this 16-key block, then this lane's row within it
    const int32_t s0 = (s.pg[sb] << log2P) + ((kb + 16 * sb) & pmask);
    const char *kbase = kpool + row_bytes_off(s0, hkv, kvh) + (int64_t)col * rowb;
#pragma unroll
    for (int st = 0; st < 4; ++st) r.k[sb][st] = __builtin_nontemporal_load((const u32x4 *)(kbase + (st * 32 + grp * 8) * 2));
    const char *vbase = vpool + row_bytes_off(s0, hkv, kvh) + (int64_t)(4 * grp) * rowb + col * 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.v[4 * sb + e] = __builtin_nontemporal_load((const u32x4 *)(vbase + e * rowb));
  }
}

// K staged in LDS (the split-KV launches of their own; the mixed launch's LDS
// belongs to the MFMA tiles, so its chunks keep the register path above).  The
// register path reads K as its MFMA operand wants it: an instruction covers 64
// bytes of each of 16 rows, which streams ~5.7 TB/s against ~7.1 TB/s for
// whole 256-byte rows (a read-only probe of both patterns over 2 KiB pool
// rows).  Here K goes to LDS the way V is read -- instruction e fills rows
// 16*(e/4) + 4*grp + e%4 of the step, 16 lanes per 256-byte row -- with
// gfx950's global-to-LDS loads, and the MFMA operands are read back with
// ds_read_b128.  LDS row q = 4e + grp holds that key; chunk c of it sits at
// c ^ swz(q % 16) (swz swaps the two 2-bit halves of its argument, an
// involution), so the 16 lanes of a group, reading one logical chunk of 16
// different keys, hit 16 different chunks: no bank conflicts.  Each wavefront
// owns two 8 KiB buffers, one per step in flight.
constexpr int kStageBytes = 2 * 32 * D * 2;  // per wavefront

__device__ __forceinline__ int kswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// s_waitcnt vmcnt(0), other counters untouched, written with the builtin so the
// compiler's own wait placement knows every earlier vector load has landed
__device__ __forceinline__ void wait_all_loads() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void dma16(const char *src, unsigned char *dst_base) {
  // dst_base: this instruction's 1 KiB of LDS; lane l lands at + 16 l.  Not
  // tracked by the compiler: the waits are explicit (see decode_item).
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)dst_base;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

__device__ __forceinline__ void load_k_lds(const SlotsSmall &s, const char *kpool, unsigned char *buf,
                                           int, int col, int grp, int, int hkv, int kvh) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    dma16(kpool + row_bytes_off(s.v[e], hkv, kvh) + 16 * (col ^ kswz(4 * (e & 3) + grp)), buf + 1024 * e);
}

__device__ __forceinline__ void load_k_lds(const SlotsBig &s, const char *kpool, unsigned char *buf,
                                           int kb, int col, int grp, int log2P, int hkv, int kvh) {
  const int pmask = (1 << log2P) - 1;
  const int64_t rowb = (int64_t)hkv * (D * 2);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int32_t s0 = (s.pg[sb] << log2P) + ((kb + 16 * sb) & pmask);
    const char *kbase = kpool + row_bytes_off(s0, hkv, kvh) + (int64_t)(4 * grp) * rowb;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dma16(kbase + e * rowb + 16 * (col ^ kswz(4 * e + grp)), buf + 1024 * (4 * sb + e));
  }
}

__device__ __forceinline__ void load_v(Regs &r, const SlotsSmall &s, const char *vpool, int, int col,
                                       int, int, int hkv, int kvh) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    r.v[e] = __builtin_nontemporal_load((const u32x4 *)(vpool + row_bytes_off(s.v[e], hkv, kvh) + col * 16));
}

__device__ __forceinline__ void load_v(Regs &r, const SlotsBig &s, const char *vpool, int kb, int col,
                                       int grp, int log2P, int hkv, int kvh) {
  const int pmask = (1 << log2P) - 1;
  const int64_t rowb = (int64_t)hkv * (D * 2);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int32_t s0 = (s.pg[sb] << log2P) + ((kb + 16 * sb) & pmask);
    const char *vbase = vpool + row_bytes_off(s0, hkv, kvh) + (int64_t)(4 * grp) * rowb + col * 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.v[4 * sb + e] = __builtin_nontemporal_load((const u32x4 *)(vbase + e * rowb));
  }
}

// K operand of key block sb, slice st for lane (col, grp): logical chunk
// 4*st + grp of key 16*sb + col, i.e. LDS row 16*sb + swz(col), chunk
// (4*st + grp) ^ col
__device__ __forceinline__ void read_k_lds(u32x4 (&kf)[2][4], const unsigned char *buf, int col,
                                           int grp) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      kf[sb][st] = *(const u32x4 *)(buf + 256 * (16 * sb + kswz(col)) + 16 * ((4 * st + grp) ^ col));
}

struct State {
  f32x4 o[8];
  float m, l;
};

__device__ __forceinline__ void step(State &st, const u32x4 (&kf)[2][4], u32x4 (&vr)[8],
                                     const bf16x8 (&qf)[4], int kb, int kend, int apos, int grp,
                                     float scale_log2) {
  f32x4 s[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) s[sb] = mfma16(as_bf16x8(kf[sb][t]), qf[t], s[sb]);
  }
  if (kb + 32 > kend) {
    // last step of the chunk: V rows of keys past the range must not reach the
    // product (their P is 0, but an unreferenced row may hold anything)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (kb + (e >> 2) * 16 + 4 * grp + (e & 3) >= kend) vr[e] = u32x4{0u, 0u, 0u, 0u};
  }
  // this lane holds column col's logits for keys kb + 16*sb + 4*grp + i
  const int rel = min(kend - 1, apos) - kb - 4 * grp;
  float x[8];
  float mx = kNegInf;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = (16 * sb + i) <= rel ? s[sb][i] : kNegInf;
      x[sb * 4 + i] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32)) * scale_log2;
  const float mn = fmaxf(st.m, mx);
  const float mu = mn == kNegInf ? 0.f : mn;
  const float al = fast_exp2(st.m - mu);
  float p[8];
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = fast_exp2(__builtin_fmaf(x[e], scale_log2, -mu));
    sum += p[e];
  }
  st.l = st.l * al + sum;
  st.m = mn;
  // P^T as B operand: slot e of lane group grp is key kb + 16*(e/4) + 4*grp + e%4,
  // the same keys the V registers hold in slot e.
  u32x4 pw;
  pw[0] = pack_bf16x2(p[0], p[1]);
  pw[1] = pack_bf16x2(p[2], p[3]);
  pw[2] = pack_bf16x2(p[4], p[5]);
  pw[3] = pack_bf16x2(p[6], p[7]);
  const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // A operand of virtual block c: channel 8*m + c of the eight keys
    const int w = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    u32x4 a;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
      a[k2] = __builtin_amdgcn_perm(vr[2 * k2 + 1][w], vr[2 * k2][w], sel);
    st.o[c] = st.o[c] * al;
    st.o[c] = mfma16(as_bf16x8(a), pf, st.o[c]);
  }
}

}  // namespace dchunk

// One wavefront runs one item.  A partial result of token t goes to partial
// row tok_pbase[t] + split, or t * pstride + split when tok_pbase is NULL.
// kst: this wavefront's kStageBytes of LDS, or NULL for the register path
template <class Slots, bool LDSK>
__device__ __forceinline__ void decode_item(const AttnArgs &a, const Item &it, unsigned char *kst) {
  using namespace dchunk;
  const int lane = threadIdx.x & 63;
  const int G = a.G;
  const int col = lane & 15, grp = lane >> 4;
  const int rows = it.ntok * G;
  const bool colv = col < rows;
  const int tl = colv ? col / G : 0;
  const int tok = it.tok0 + tl;
  const int qh = it.kvh * G + (colv ? col % G : 0);
  const int apos = it.pos0 + tl;

  bf16x8 qf[4];
  {
    const uint16_t *qrow = (const uint16_t *)a.q + ((int64_t)tok * a.Hq + qh) * D;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 v = *(const u32x4 *)(qrow + t * 32 + grp * 8);
      if (!colv) v = u32x4{0u, 0u, 0u, 0u};
      qf[t] = as_bf16x8(v);
    }
  }
  State st;
#pragma unroll
  for (int c = 0; c < 8; ++c) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.f;

  const int32_t *ptrow = a.page_table + (int64_t)it.req * a.pt_stride;
  const char *kp = (const char *)a.kpool;
  const char *vp = (const char *)a.vpool;
  const int kend = it.kend;
  const int L2 = a.log2P;
  Slots sa, sb;
  Regs ra, rb;
  if (LDSK) {
    // Steps alternate between the two LDS buffers and register sets.  A step
    // first waits for everything in flight (its own K rows in LDS and V rows in
    // registers), then issues the next step's loads, then reads its K operands
    // and computes, so one step of loads is always in flight during the math.
    // (The K loads are not tracked by the compiler; the waits below are
    // explicit, and the compiler sees them, so it adds none of its own for the
    // V registers.)
    unsigned char *kb0 = kst, *kb1 = kst + kStageBytes / 2;
    u32x4 kf[2][4];
    lookup(sa, ptrow, it.kbeg, kend, col, grp, L2, a.num_pages);
    load_v(ra, sa, vp, it.kbeg, col, grp, L2, a.Hkv, it.kvh);
    load_k_lds(sa, kp, kb0, it.kbeg, col, grp, L2, a.Hkv, it.kvh);
    if (it.kbeg + kDecodeKeys < kend)
      lookup(sb, ptrow, it.kbeg + kDecodeKeys, kend, col, grp, L2, a.num_pages);
    for (int kb = it.kbeg; kb < kend; kb += 2 * kDecodeKeys) {
      wait_all_loads();
      if (kb + kDecodeKeys < kend) {
        load_v(rb, sb, vp, kb + kDecodeKeys, col, grp, L2, a.Hkv, it.kvh);
        load_k_lds(sb, kp, kb1, kb + kDecodeKeys, col, grp, L2, a.Hkv, it.kvh);
      }
      if (kb + 2 * kDecodeKeys < kend)
        lookup(sa, ptrow, kb + 2 * kDecodeKeys, kend, col, grp, L2, a.num_pages);
      read_k_lds(kf, kb0, col, grp);
      step(st, kf, ra.v, qf, kb, kend, apos, grp, a.scale_log2);
      if (kb + kDecodeKeys >= kend) break;
      wait_all_loads();
      if (kb + 2 * kDecodeKeys < kend) {
        load_v(ra, sa, vp, kb + 2 * kDecodeKeys, col, grp, L2, a.Hkv, it.kvh);
        load_k_lds(sa, kp, kb0, kb + 2 * kDecodeKeys, col, grp, L2, a.Hkv, it.kvh);
      }
      if (kb + 3 * kDecodeKeys < kend)
        lookup(sb, ptrow, kb + 3 * kDecodeKeys, kend, col, grp, L2, a.num_pages);
      read_k_lds(kf, kb1, col, grp);
      step(st, kf, rb.v, qf, kb + kDecodeKeys, kend, apos, grp, a.scale_log2);
    }
    // no load may outlive the wavefront's use of its buffers
    wait_all_loads();
  } else {
    lookup(sa, ptrow, it.kbeg, kend, col, grp, L2, a.num_pages);
    load(ra, sa, kp, vp, it.kbeg, col, grp, L2, a.Hkv, it.kvh);
    if (it.kbeg + kDecodeKeys < kend)
      lookup(sb, ptrow, it.kbeg + kDecodeKeys, kend, col, grp, L2, a.num_pages);
    for (int kb = it.kbeg; kb < kend; kb += 2 * kDecodeKeys) {
      if (kb + kDecodeKeys < kend) load(rb, sb, kp, vp, kb + kDecodeKeys, col, grp, L2, a.Hkv, it.kvh);
      if (kb + 2 * kDecodeKeys < kend)
        lookup(sa, ptrow, kb + 2 * kDecodeKeys, kend, col, grp, L2, a.num_pages);
      step(st, ra.k, ra.v, qf, kb, kend, apos, grp, a.scale_log2);
      if (kb + kDecodeKeys >= kend) break;
      if (kb + 2 * kDecodeKeys < kend)
        load(ra, sa, kp, vp, kb + 2 * kDecodeKeys, col, grp, L2, a.Hkv, it.kvh);
      if (kb + 3 * kDecodeKeys < kend)
        lookup(sb, ptrow, kb + 3 * kDecodeKeys, kend, col, grp, L2, a.num_pages);
      step(st, rb.k, rb.v, qf, kb + kDecodeKeys, kend, apos, grp, a.scale_log2);
    }
  }

  float l = st.l;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (!colv) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  // O^T block c: this lane holds channels 8*(4*grp + i) + c, i < 4, c < 8
  if (it.split < 0) {
    uint16_t *orow = (uint16_t *)a.out + ((int64_t)tok * a.Hq + qh) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 w;
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2)
        w[c2] = pack_bf16x2(st.o[2 * c2][i] * inv, st.o[2 * c2 + 1][i] * inv);
      *(u32x4 *)(orow + 8 * (4 * grp + i)) = w;
    }
  } else {
    const int64_t pi = (a.tok_pbase ? (int64_t)a.tok_pbase[tok] : (int64_t)tok * a.pstride) + it.split;
    float *prow = a.o_part + (pi * a.Hq + qh) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 w0, w1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        w0[c] = st.o[c][i] * inv;
        w1[c] = st.o[c + 4][i] * inv;
      }
      *(f32x4 *)(prow + 8 * (4 * grp + i)) = w0;
      *(f32x4 *)(prow + 8 * (4 * grp + i) + 4) = w1;
    }
    if (grp == 0) a.lse_part[pi * a.Hq + qh] = l > 0.f ? st.m + fast_log2(l) : kNegInf;
  }
}

// One wavefront of a WPB-wavefront block runs item block*WPB + wave of the list.
// stage: the block's WPB * kStageBytes of LDS for staged K, or NULL.
template <class Slots, int WPB = kDecodeWavesPerBlock>
__device__ __forceinline__ void decode_chunk(const AttnArgs &a, int block, unsigned char *stage = nullptr) {
  // uniform wavefront index: the item and its page ids are then scalar loads,
  // which do not wait on the vector-load counter of the K/V loads in flight
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ii = block * WPB + wave;
  if (ii >= a.n_items) return;
  const Item it = a.items[ii];
  if (it.ntok == 0) return;
  if (stage)
    decode_item<Slots, true>(a, it, stage + wave * dchunk::kStageBytes);
  else
    decode_item<Slots, false>(a, it, nullptr);
}

}  // namespace rpkv
