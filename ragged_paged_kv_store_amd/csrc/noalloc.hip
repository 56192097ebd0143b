// rpkv_graph_decode_forward_noalloc: the graph-capturable decode step for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  It runs the kernels of
// rpkv_graph_decode_forward (store_kv, split-KV chunks, log-sum-exp merge) with
// the split-KV partials in a fixed file-scope device array instead of buffers
// allocated by rpkv_graph_decode_init, so it needs no init and calls no
// allocating routine.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>

#include "plan_state.h"

// Partials of one call: [rows, D] fp32 normalised outputs, then [rows] fp32
// base-2 log-sum-exps (each part 256-byte aligned), rows = batch * q_len *
// chunks * Hq.  Each GPU the library runs on holds its own copy until the
// process ends; every call on a GPU reuses it.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_scratch[kMaxDevices];
int g_scratch_err[kMaxDevices];

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The array's address on device `dev` (the current device), looked up once per
// device; host code uses this address, never the array's name.
int scratch_address(int dev, void **ptr) {
  std::call_once(g_once[dev], [dev] {
    g_scratch_err[dev] = (int)hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  *ptr = g_scratch[dev];
  return g_scratch_err[dev];
}

}  // namespace

using rpkv::fail;
using rpkv::hip_fail;

extern "C" rpkv_status rpkv_graph_decode_forward_noalloc(
    rpkv_plan *p, int32_t batch, int32_t q_len, int32_t max_seq_len, const void *q, const void *k,
    const void *v, const int32_t *slot_mapping, void *kpool, void *vpool, const int32_t *seq_lens,
    const int32_t *page_table, int64_t pt_stride, int32_t pt_cols, void *out, float scale,
    void *stream) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (p->s.dtype != RPKV_BF16) return fail(RPKV_ERR_UNSUPPORTED, "graph decode is bf16 only");
  if (batch < 0 || q_len < 1 || max_seq_len < q_len)
    return fail(RPKV_ERR_INVALID_ARG, "need batch >= 0, q_len >= 1, max_seq_len >= q_len");
  if ((int64_t)q_len * p->s.G() > rpkv::kDecodeRows)
    return fail(RPKV_ERR_UNSUPPORTED, "q_len * Hq / Hkv must be <= 16 (one split-KV item)");
  if (batch > p->s.max_batch || (int64_t)batch * q_len > p->s.max_tokens)
    return fail(RPKV_ERR_CAPACITY, "batch exceeds the plan's max_batch or max_tokens");
  if ((int64_t)max_seq_len > (int64_t)p->s.max_pages_per_req * p->s.P)
    return fail(RPKV_ERR_CAPACITY, "max_seq_len exceeds max_pages_per_req * page_size");
  if (batch == 0) return RPKV_OK;
  if (!q || !k || !v || !slot_mapping || !kpool || !vpool || !seq_lens || !page_table || !out)
    return fail(RPKV_ERR_INVALID_ARG,
                "q, k, v, slot_mapping, pools, seq_lens, page_table, out must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)kpool | (uintptr_t)vpool |
       (uintptr_t)out) & 15)
    return fail(RPKV_ERR_INVALID_ARG, "q, k, v, pools and out must be 16-byte aligned");
  if (pt_cols < 0 || pt_stride < pt_cols || (int64_t)pt_cols * p->s.P < (int64_t)max_seq_len)
    return fail(RPKV_ERR_INVALID_ARG, "page table must have ceil(max_seq_len / page_size) columns");
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(RPKV_ERR_INVALID_ARG, "scale must be finite and positive");
  // the chunking rpkv_graph_decode_init would pick for max_batch = batch
  int32_t chunk = 0, maxc = 0;
  rpkv::graph_decode_chunks(batch, p->s.Hkv, max_seq_len, &chunk, &maxc);
  const size_t rows = (size_t)batch * q_len * maxc * p->s.Hq;
  const size_t obytes = align256(rows * p->s.D * sizeof(float));
  const size_t need = maxc > 1 ? obytes + align256(rows * sizeof(float)) : 0;
  if (need > kScratchBytes)
    return fail(RPKV_ERR_CAPACITY,
                "the batch's split-KV partials need " + std::to_string(need) +
                    " bytes; the no-alloc scratch holds " + std::to_string(kScratchBytes) +
                    " (fewer requests or a shorter max_seq_len per call)");
  int dev = 0;
  int e = hipGetDevice(&dev);
  if (e) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RPKV_ERR_UNSUPPORTED, "device index beyond the no-alloc scratch table");
  void *base = nullptr;
  e = scratch_address(dev, &base);
  if (e) return hip_fail(e, "hipGetSymbolAddress (no-alloc scratch)");

  const int32_t T = batch * q_len;
  const int64_t row_bytes = (int64_t)p->s.Hkv * p->s.D * 2;
  const int64_t num_slots = p->s.num_pages * p->s.P;
  rpkv_status st = rpkv::timed(p, RPKV_KERNEL_STORE, stream, [&] {
    return rpkv::launch_store_kv(k, v, slot_mapping, T, row_bytes, num_slots, kpool, vpool, stream);
  }, "store_kv launch");
  if (st != RPKV_OK) return st;
  rpkv::AttnArgs a{};
  a.q = q;
  a.kpool = kpool;
  a.vpool = vpool;
  a.out = out;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.tok_pbase = nullptr;
  a.pstride = maxc;
  a.o_part = (float *)base;
  a.lse_part = (float *)((char *)base + obytes);
  a.Hq = p->s.Hq;
  a.Hkv = p->s.Hkv;
  a.G = p->s.G();
  a.D = p->s.D;
  a.log2P = p->s.log2P;
  a.num_pages = p->s.num_pages;
  a.scale_log2 = scale * 1.4426950408889634f;
  st = rpkv::timed(p, RPKV_KERNEL_DECODE, stream, [&] {
    return rpkv::launch_graph_decode_bf16(a, seq_lens, q_len, chunk, maxc, max_seq_len, batch,
                                          stream);
  }, "graph decode launch");
  if (st != RPKV_OK || maxc <= 1) return st;
  return rpkv::timed(p, RPKV_KERNEL_MERGE, stream, [&] {
    return rpkv::launch_graph_merge(seq_lens, q_len, chunk, maxc, max_seq_len, T, a.o_part,
                                    a.lse_part, out, p->s.Hq, p->s.D, p->s.dtype, stream);
  }, "graph merge launch");
}
