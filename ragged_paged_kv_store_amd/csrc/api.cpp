// C ABI (include/rpkv.h): argument checks, per-batch metadata upload and the
// per-layer launch sequence store_kv -> tiles -> split-KV chunks -> merge.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "plan_state.h"

using rpkv::HostPlan;
using rpkv::Item;
using rpkv::Shape;

namespace {

// Opt-in plan log: RPKV_LOG_PLANS set to anything but "0" prints each
// successful plan's summary line to stderr.
bool log_plans() {
  static const bool on = [] {
    const char *v = std::getenv("RPKV_LOG_PLANS");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}
thread_local std::string g_err;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

namespace rpkv {
rpkv_status fail(rpkv_status st, const std::string &msg) {
  g_err = msg;
  return st;
}

rpkv_status hip_fail(int err, const char *what) {
  return fail(RPKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString((hipError_t)err));
}
}  // namespace rpkv

using rpkv::fail;
using rpkv::hip_fail;
using rpkv::timed;


namespace {

size_t workspace_need(const rpkv_plan *p) {
  if (p->hp.n_partials == 0) return 0;
  const size_t rows = (size_t)p->hp.n_partials * p->s.Hq;
  return align256(rows * p->s.D * sizeof(float)) + align256(rows * sizeof(float));
}

// Frees the plan's metadata buffers (the caller has waited for the device).
void release_device(rpkv_plan *p) {
  if (p->dmeta) (void)hipFree(p->dmeta);
  if (p->csr_table) (void)hipFree(p->csr_table);
  p->dmeta = nullptr;
  p->csr_table = nullptr;
  for (int i = 0; i < 2; ++i) {
    if (p->hmeta[i]) (void)hipHostFree(p->hmeta[i]);
    if (p->hev[i]) (void)hipEventDestroy(p->hev[i]);
    p->hmeta[i] = nullptr;
    p->hev[i] = nullptr;
    p->hev_live[i] = false;
  }
  p->device = -1;
}


}  // namespace

extern "C" {

const char *rpkv_status_string(rpkv_status st) {
  switch (st) {
    case RPKV_OK: return "RPKV_OK";
    case RPKV_ERR_INVALID_ARG: return "RPKV_ERR_INVALID_ARG";
    case RPKV_ERR_UNSUPPORTED: return "RPKV_ERR_UNSUPPORTED";
    case RPKV_ERR_WORKSPACE_TOO_SMALL: return "RPKV_ERR_WORKSPACE_TOO_SMALL";
    case RPKV_ERR_NOT_PREPARED: return "RPKV_ERR_NOT_PREPARED";
    case RPKV_ERR_HIP: return "RPKV_ERR_HIP";
    case RPKV_ERR_CAPACITY: return "RPKV_ERR_CAPACITY";
  }
  return "RPKV_ERR_UNKNOWN";
}

const char *rpkv_last_error(void) { return g_err.c_str(); }

rpkv_status rpkv_supports(const rpkv_shape *shape) {
  Shape s;
  std::string msg;
  rpkv_status st = rpkv::check_shape(shape, &s, &msg);
  if (st != RPKV_OK) return fail(st, msg);
  return RPKV_OK;
}

rpkv_status rpkv_plan_create(const rpkv_shape *shape, rpkv_plan **out) {
  if (!out) return fail(RPKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  Shape s;
  std::string msg;
  rpkv_status st = rpkv::check_shape(shape, &s, &msg);
  if (st != RPKV_OK) return fail(st, msg);
  rpkv_plan *p = new (std::nothrow) rpkv_plan();
  if (!p) return fail(RPKV_ERR_CAPACITY, "host allocation failed");
  p->s = s;
  p->meta_cap = rpkv::meta_layout(rpkv::meta_caps(s)).bytes;
  *out = p;
  return RPKV_OK;
}

void rpkv_plan_destroy(rpkv_plan *p) {
  if (!p) return;
  if (p->dmeta || p->hmeta[0] || p->hmeta[1] || !p->ev.empty() || p->g_opart) {
    if (p->device >= 0) (void)hipSetDevice(p->device);
    else if (p->g_device >= 0) (void)hipSetDevice(p->g_device);
    (void)hipDeviceSynchronize();
  }
  release_device(p);
  if (p->g_opart) (void)hipFree(p->g_opart);
  for (hipEvent_t e : p->ev) (void)hipEventDestroy(e);
  delete p;
}

rpkv_status rpkv_plan_batch(rpkv_plan *p, int32_t batch, const int32_t *cu, const int32_t *seqlens,
                            int32_t cols, const int32_t *pt_host, const rpkv_prefix_group *groups,
                            int32_t ngroups) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  p->prepared = false;
  p->planned = false;
  std::string msg;
  rpkv_status st;
  try {
    st = rpkv::plan_batch_host(p->s, batch, cu, seqlens, cols, pt_host, groups, ngroups,
                               &p->hp_next, &msg);
  } catch (const std::bad_alloc &) {
    return fail(RPKV_ERR_CAPACITY, "host allocation failed while planning");
  }
  if (st != RPKV_OK) return fail(st, msg);
  const rpkv::MetaLayout lay = rpkv::meta_layout(rpkv::meta_counts(p->hp_next, p->s.max_batch));
  if (lay.bytes > p->meta_cap)  // the bound of meta_caps is exceeded: a planner bug
    return fail(RPKV_ERR_CAPACITY, "work partition of " + std::to_string(lay.bytes) +
                                       " bytes exceeds the plan's metadata capacity of " +
                                       std::to_string(p->meta_cap));
  std::swap(p->hp, p->hp_next);
  p->lay = lay;
  p->planned = true;
  p->ws_need = workspace_need(p);
  if (log_plans()) {
    char line[512];
    if (rpkv_plan_summary(p, line, sizeof line) == RPKV_OK) std::fprintf(stderr, "rpkv: %s\n", line);
  }
  return RPKV_OK;
}

rpkv_status rpkv_plan_summary(const rpkv_plan *p, char *buf, size_t size) {
  if (!p || !buf || size == 0) return fail(RPKV_ERR_INVALID_ARG, "plan or buffer is NULL or empty");
  if (!p->planned) return fail(RPKV_ERR_NOT_PREPARED, "no planned batch");
  const HostPlan &hp = p->hp;
  int32_t ndec_req = 0, npre_req = 0, nempty = 0;
  for (int32_t i = 0; i < hp.batch; ++i) {
    const int32_t n = hp.cu_q[i + 1] - hp.cu_q[i];
    if (n == 0) ++nempty;
    else if ((int64_t)n * p->s.G() <= p->s.decode_max_rows) ++ndec_req;
    else ++npre_req;
  }
  int64_t nm = 0;
  for (const rpkv::CascNode &nd : hp.tree) nm += (int64_t)nd.members.size();
  std::snprintf(buf, size,
                "batch %d (%d tokens): %d decode-type, %d prefill-type, %d empty requests; "
                "%d MFMA tiles (%d per workgroup, %d in shared-prefix levels), %zu split-KV "
                "chunks of %d keys; %zu cascade levels (depth %d, %lld member entries, %d "
                "requests); %lld partials, %zu tokens merged; metadata %zu bytes; planned "
                "in %.1f us",
                hp.batch, hp.T, ndec_req, npre_req, nempty, hp.n_prefill_real, hp.tiles_per_block,
                hp.n_cascade_items, hp.decode.size(), hp.decode_chunk, hp.tree.size(),
                hp.cascade_depth, (long long)nm, hp.cascade_members, (long long)hp.n_partials,
                hp.merge.size() / 3, p->lay.bytes, hp.plan_us);
  return RPKV_OK;
}

namespace {

// The plan's device buffers and pinned staging, allocated once on the device of
// the first prepare, at the capacity every batch fits in: the per-batch path
// never allocates, frees or synchronises the device for memory.
rpkv_status ensure_device(rpkv_plan *p) {
  int dev = 0;
  int e = hipGetDevice(&dev);
  if (e) return hip_fail(e, "hipGetDevice");
  if (p->device >= 0) {
    if (p->device != dev)
      return fail(RPKV_ERR_INVALID_ARG, "a plan is bound to the device of its first prepare");
    return RPKV_OK;
  }
  const size_t csr_bytes =
      std::max<size_t>(1, (size_t)p->s.max_batch * p->s.max_pages_per_req) * sizeof(int32_t);
  const char *what = nullptr;
  if ((e = hipMalloc((void **)&p->dmeta, p->meta_cap))) what = "hipMalloc (plan metadata)";
  else if ((e = hipMalloc((void **)&p->csr_table, csr_bytes)))
    what = "hipMalloc (dense copy of a CSR page table)";
  else p->n_alloc += 2;
  for (int i = 0; !what && i < 2; ++i) {
    if ((e = hipHostMalloc((void **)&p->hmeta[i], p->meta_cap, hipHostMallocDefault)))
      what = "hipHostMalloc (metadata staging)";
    else if ((e = hipEventCreateWithFlags(&p->hev[i], hipEventDisableTiming)))
      what = "hipEventCreate";
    else ++p->n_alloc;
  }
  if (what) {
    const rpkv_status st = hip_fail(e, what);
    release_device(p);
    return st;
  }
  p->device = dev;
  return RPKV_OK;
}

// prepare_metadata; csr_indptr (a CSR page table's row offsets) rides along in
// the metadata upload
rpkv_status prepare_impl(rpkv_plan *p, int32_t batch, const int32_t *cu, const int32_t *seqlens,
                         const int32_t *pt_dev, int64_t pt_stride, int32_t cols,
                         const int32_t *pt_host, const rpkv_prefix_group *groups, int32_t ngroups,
                         void *ws, size_t ws_bytes, void *stream,
                         const std::vector<int32_t> *csr_indptr) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (pt_stride < cols) return fail(RPKV_ERR_INVALID_ARG, "page_table_stride < page_table_cols");
  rpkv_status st = rpkv_plan_batch(p, batch, cu, seqlens, cols, pt_host, groups, ngroups);
  if (st != RPKV_OK) return st;
  if (csr_indptr)
    p->hp.csr_indptr = *csr_indptr;
  else
    p->hp.csr_indptr.clear();
  p->planned = false;  // becomes usable only once uploaded
  const HostPlan &hp = p->hp;
  bool any_keys = false;
  for (int32_t i = 0; i < batch; ++i) any_keys |= seqlens[i] > 0 && cu[i + 1] > cu[i];
  if (any_keys && !pt_dev) return fail(RPKV_ERR_INVALID_ARG, "page_table_dev is NULL");
  if (p->ws_need > 0) {
    if (!ws || ws_bytes < p->ws_need)
      return fail(RPKV_ERR_WORKSPACE_TOO_SMALL,
                  "workspace of " + std::to_string(p->ws_need) + " bytes needed, " +
                      std::to_string(ws ? ws_bytes : 0) + " given");
    if ((uintptr_t)ws & 255) return fail(RPKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  rpkv_status dst = ensure_device(p);
  if (dst != RPKV_OK) return dst;
  const rpkv::MetaLayout &lay = p->lay;
  const int c = p->hcur;
  int e = 0;
  if (p->hev_live[c]) {  // the upload that last used this staging buffer
    e = hipEventSynchronize(p->hev[c]);
    if (e) return hip_fail(e, "hipEventSynchronize");
    p->hev_live[c] = false;
  }
  char *h = p->hmeta[c];
  const size_t bytes = lay.bytes;
  std::memset(h, 0, bytes);
  if (!hp.prefill.empty()) std::memcpy(h + lay.off_pre, hp.prefill.data(), hp.prefill.size() * sizeof(Item));
  if (!hp.decode.empty()) std::memcpy(h + lay.off_dec, hp.decode.data(), hp.decode.size() * sizeof(Item));
  if (!hp.tok_pbase.empty())
    std::memcpy(h + lay.off_pbase, hp.tok_pbase.data(), hp.tok_pbase.size() * sizeof(int32_t));
  if (!hp.merge.empty()) std::memcpy(h + lay.off_merge, hp.merge.data(), hp.merge.size() * sizeof(int32_t));
  if (!hp.toklist.empty())
    std::memcpy(h + lay.off_tok, hp.toklist.data(), hp.toklist.size() * sizeof(int32_t));
  if (!hp.csr_indptr.empty())
    std::memcpy(h + lay.off_indptr, hp.csr_indptr.data(), hp.csr_indptr.size() * sizeof(int32_t));
  e = hipMemcpyAsync(p->dmeta, h, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e) return hip_fail(e, "hipMemcpyAsync (metadata)");
  e = hipEventRecord(p->hev[c], (hipStream_t)stream);
  if (e) return hip_fail(e, "hipEventRecord");
  p->hev_live[c] = true;
  p->hcur ^= 1;
  p->page_table = pt_dev;
  p->pt_stride = pt_stride;
  if (p->ws_need > 0) {
    const size_t rows = (size_t)hp.n_partials * p->s.Hq;
    p->o_part = (float *)ws;
    p->lse_part = (float *)((char *)ws + align256(rows * p->s.D * sizeof(float)));
  } else {
    p->o_part = p->lse_part = nullptr;
  }
  p->planned = true;
  p->prepared = true;
  return RPKV_OK;
}

}  // namespace

rpkv_status rpkv_prepare_metadata(rpkv_plan *p, int32_t batch, const int32_t *cu,
                                  const int32_t *seqlens, const int32_t *pt_dev, int64_t pt_stride,
                                  int32_t cols, const int32_t *pt_host,
                                  const rpkv_prefix_group *groups, int32_t ngroups, void *ws,
                                  size_t ws_bytes, void *stream) {
  return prepare_impl(p, batch, cu, seqlens, pt_dev, pt_stride, cols, pt_host, groups, ngroups, ws,
                      ws_bytes, stream, nullptr);
}

rpkv_status rpkv_prepare_metadata_csr(rpkv_plan *p, int32_t batch, const int32_t *cu,
                                      const int32_t *indptr, const int32_t *last_page_len,
                                      const int32_t *indices_dev, const int32_t *indices_host,
                                      const rpkv_prefix_group *groups, int32_t ngroups, void *ws,
                                      size_t ws_bytes, void *stream) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (batch < 0) return fail(RPKV_ERR_INVALID_ARG, "batch < 0");
  if (batch > p->s.max_batch) return fail(RPKV_ERR_CAPACITY, "batch exceeds max_batch");
  if (batch > 0 && (!indptr || !last_page_len || !cu))
    return fail(RPKV_ERR_INVALID_ARG, "cu_seqlens_q, page_indptr and last_page_len must be non-NULL");
  if (batch > 0 && indptr[0] != 0) return fail(RPKV_ERR_INVALID_ARG, "page_indptr[0] must be 0");
  const int32_t P = p->s.P;
  std::vector<int32_t> L(batch), iptr(batch > 0 ? indptr : nullptr, batch > 0 ? indptr + batch + 1 : nullptr);
  int32_t cols = 1;
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t pages = indptr[i + 1] - indptr[i];
    if (pages < 0) return fail(RPKV_ERR_INVALID_ARG, "page_indptr must be non-decreasing");
    if (pages > p->s.max_pages_per_req)
      return fail(RPKV_ERR_CAPACITY, "a request has more pages than max_pages_per_req");
    if (pages > 0 && (last_page_len[i] < 1 || last_page_len[i] > P))
      return fail(RPKV_ERR_INVALID_ARG, "last_page_len must be in [1, page_size]");
    L[i] = pages > 0 ? (pages - 1) * P + last_page_len[i] : 0;
    cols = std::max(cols, pages);
  }
  const int32_t total = batch > 0 ? indptr[batch] : 0;
  if (total > 0 && !indices_dev) return fail(RPKV_ERR_INVALID_ARG, "page_indices_dev is NULL");
  std::vector<int32_t> host;
  if (indices_host) {
    host.assign((size_t)batch * cols, 0);
    for (int32_t i = 0; i < batch; ++i)
      std::memcpy(host.data() + (size_t)i * cols, indices_host + indptr[i],
                  (size_t)(indptr[i + 1] - indptr[i]) * sizeof(int32_t));
  }
  rpkv_status dst = ensure_device(p);
  if (dst != RPKV_OK) return dst;
  rpkv_status st = prepare_impl(p, batch, cu, L.data(), p->csr_table, p->s.max_pages_per_req, cols,
                                indices_host ? host.data() : nullptr, groups, ngroups, ws, ws_bytes,
                                stream, &iptr);
  if (st != RPKV_OK) return st;
  // expand the rows on the stream, after the upload of the offsets
  const int e = rpkv::launch_csr_to_dense(batch, (const int32_t *)(p->dmeta + p->lay.off_indptr),
                                          indices_dev, p->csr_table, p->s.max_pages_per_req, stream);
  if (e) {
    p->prepared = false;
    return hip_fail(e, "csr_to_dense launch");
  }
  return RPKV_OK;
}

rpkv_status rpkv_rewrite_block_table(int32_t batch, const int32_t *table, int64_t stride,
                                     int32_t cols, int32_t factor, int32_t *out,
                                     int64_t out_stride, void *stream) {
  if (batch < 0 || cols < 0 || factor < 1)
    return fail(RPKV_ERR_INVALID_ARG, "need batch >= 0, cols >= 0, factor >= 1");
  if (stride < cols || out_stride < (int64_t)cols * factor || (int64_t)cols * factor > INT32_MAX)
    return fail(RPKV_ERR_INVALID_ARG, "need stride >= cols and out_stride >= cols * factor");
  if (batch > 0 && cols > 0 && (!table || !out))
    return fail(RPKV_ERR_INVALID_ARG, "table and out must be non-NULL");
  const int e = rpkv::launch_rewrite_blocks(batch, table, stride, cols, factor, out, out_stride, stream);
  if (e) return hip_fail(e, "rewrite_block_table launch");
  return RPKV_OK;
}

rpkv_status rpkv_workspace_bytes(const rpkv_plan *p, size_t *bytes) {
  if (!p || !bytes) return fail(RPKV_ERR_INVALID_ARG, "plan or bytes is NULL");
  *bytes = p->ws_need;
  return RPKV_OK;
}

rpkv_status rpkv_last_indices(const rpkv_plan *p, int32_t *out) {
  if (!p || !out) return fail(RPKV_ERR_INVALID_ARG, "plan or out is NULL");
  if (!p->planned) return fail(RPKV_ERR_NOT_PREPARED, "no planned batch");
  for (int32_t i = 0; i < p->hp.batch; ++i)
    out[i] = p->hp.cu_q[i + 1] > p->hp.cu_q[i] ? p->hp.cu_q[i + 1] - 1 : -1;
  return RPKV_OK;
}

rpkv_status rpkv_plan_get_info(const rpkv_plan *p, rpkv_plan_info *info) {
  if (!p || !info) return fail(RPKV_ERR_INVALID_ARG, "plan or info is NULL");
  if (!p->planned) return fail(RPKV_ERR_NOT_PREPARED, "no planned batch");
  const HostPlan &hp = p->hp;
  info->batch = hp.batch;
  info->num_tokens = hp.T;
  info->max_seqlen_q = hp.max_q;
  info->max_seqlen_k = hp.max_k;
  info->num_prefill_items = hp.n_prefill_real;
  info->num_decode_items = (int32_t)hp.decode.size();
  info->num_cascade_items = hp.n_cascade_items;
  info->num_merge_tokens = (int32_t)(hp.merge.size() / 3);
  info->num_partials = hp.n_partials;
  info->workspace_bytes = (int64_t)p->ws_need;
  info->decode_chunk = hp.decode_chunk;
  info->cascade_members = hp.cascade_members;
  info->plan_host_us = hp.plan_us;
  info->num_cascade_levels = (int32_t)hp.tree.size();
  info->cascade_depth = hp.cascade_depth;
  int64_t nm = 0;
  for (const rpkv::CascNode &nd : hp.tree) nm += (int64_t)nd.members.size();
  info->num_cascade_level_members = (int32_t)nm;
  info->tiles_per_block = hp.tiles_per_block;
  info->metadata_bytes = (int64_t)p->lay.bytes;
  info->metadata_capacity_bytes = (int64_t)p->meta_cap;
  info->buffer_allocations = p->n_alloc;
  return RPKV_OK;
}

rpkv_status rpkv_plan_get_cascade_tree(const rpkv_plan *p, int32_t max_levels, int32_t max_members,
                                       int32_t *parent, int32_t *prefix, int32_t *indptr,
                                       int32_t *members) {
  if (!p || max_levels < 0 || max_members < 0)
    return fail(RPKV_ERR_INVALID_ARG, "bad arguments to rpkv_plan_get_cascade_tree");
  if (!p->planned) return fail(RPKV_ERR_NOT_PREPARED, "no planned batch");
  const std::vector<rpkv::CascNode> &tree = p->hp.tree;
  int64_t nm = 0;
  for (const rpkv::CascNode &nd : tree) nm += (int64_t)nd.members.size();
  if ((int64_t)tree.size() > max_levels || nm > max_members)
    return fail(RPKV_ERR_CAPACITY, "cascade tree has " + std::to_string(tree.size()) +
                                       " levels and " + std::to_string(nm) + " member entries");
  if (!indptr || (!tree.empty() && (!parent || !prefix || !members)))
    return fail(RPKV_ERR_INVALID_ARG, "output arrays must be non-NULL");
  int32_t o = 0;
  indptr[0] = 0;
  for (size_t k = 0; k < tree.size(); ++k) {
    parent[k] = tree[k].parent;
    prefix[k] = tree[k].prefix;
    for (int32_t j : tree[k].members) members[o++] = j;
    indptr[k + 1] = o;
  }
  return RPKV_OK;
}

rpkv_status rpkv_plan_get_items(const rpkv_plan *p, int32_t kind, int32_t *items, int32_t capacity,
                                int32_t *count) {
  if (!p || !count || (kind != 0 && kind != 1) || capacity < 0 || (capacity > 0 && !items))
    return fail(RPKV_ERR_INVALID_ARG, "bad arguments to rpkv_plan_get_items");
  if (!p->planned) return fail(RPKV_ERR_NOT_PREPARED, "no planned batch");
  const std::vector<Item> &v = kind == 0 ? p->hp.prefill : p->hp.decode;
  *count = (int32_t)v.size();
  const int32_t n = std::min<int32_t>(capacity, (int32_t)v.size());
  if (n > 0) std::memcpy(items, v.data(), (size_t)n * sizeof(Item));
  return RPKV_OK;
}

rpkv_status rpkv_plan_get_token_list(const rpkv_plan *p, int32_t *out, int32_t capacity,
                                     int32_t *count) {
  if (!p || !count || capacity < 0 || (capacity > 0 && !out))
    return fail(RPKV_ERR_INVALID_ARG, "bad arguments to rpkv_plan_get_token_list");
  if (!p->planned) return fail(RPKV_ERR_NOT_PREPARED, "no planned batch");
  *count = (int32_t)p->hp.toklist.size();
  const int32_t n = std::min<int32_t>(capacity, *count);
  if (n > 0) std::memcpy(out, p->hp.toklist.data(), (size_t)n * sizeof(int32_t));
  return RPKV_OK;
}

rpkv_status rpkv_store_kv(rpkv_plan *p, const void *k, const void *v, const int32_t *slots,
                          int64_t T, void *kpool, void *vpool, void *stream) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (T < 0) return fail(RPKV_ERR_INVALID_ARG, "num_tokens < 0");
  if (T == 0) return RPKV_OK;
  if (!k || !v || !slots || !kpool || !vpool)
    return fail(RPKV_ERR_INVALID_ARG, "k, v, slot_mapping and pools must be non-NULL");
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)kpool | (uintptr_t)vpool) & 15)
    return fail(RPKV_ERR_INVALID_ARG, "k, v and pools must be 16-byte aligned");
  const int64_t row_bytes = (int64_t)p->s.Hkv * p->s.D * (p->s.dtype == RPKV_BF16 ? 2 : 4);
  const int64_t num_slots = p->s.num_pages * p->s.P;
  if (p->s.check_slots) {
    // debug mode: read the slots back once the stream has produced them
    p->slots_host.resize((size_t)T);
    int e = hipMemcpyAsync(p->slots_host.data(), slots, (size_t)T * sizeof(int32_t),
                           hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (!e) e = hipStreamSynchronize((hipStream_t)stream);
    if (e) return hip_fail(e, "copying slot_mapping to the host (check_slots)");
    std::string msg;
    if (rpkv::find_bad_slot(p->slots_host.data(), T, num_slots, &p->slots_key, &msg) >= 0)
      return fail(RPKV_ERR_INVALID_ARG, msg);
  }
  return timed(p, RPKV_KERNEL_STORE, stream, [&] {
    return rpkv::launch_store_kv(k, v, slots, T, row_bytes, num_slots, kpool, vpool, stream);
  }, "store_kv launch");
}

rpkv_status rpkv_check_slot_mapping(const rpkv_plan *p, const int32_t *slots, int64_t T) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (T < 0 || (T > 0 && !slots)) return fail(RPKV_ERR_INVALID_ARG, "need num_tokens >= 0 and slots");
  if (T > INT32_MAX) return fail(RPKV_ERR_INVALID_ARG, "num_tokens exceeds int32");
  std::vector<int64_t> key;
  std::string msg;
  if (rpkv::find_bad_slot(slots, T, p->s.num_pages * p->s.P, &key, &msg) >= 0)
    return fail(RPKV_ERR_INVALID_ARG, msg);
  return RPKV_OK;
}

rpkv_status rpkv_attend(rpkv_plan *p, const void *q, const void *kpool, const void *vpool,
                        void *out, float scale, void *stream) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (!p->prepared) return fail(RPKV_ERR_NOT_PREPARED, "attend before a successful prepare_metadata");
  const HostPlan &hp = p->hp;
  if (hp.T == 0) return RPKV_OK;
  if (!q || !kpool || !vpool || !out)
    return fail(RPKV_ERR_INVALID_ARG, "q, pools and out must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)kpool | (uintptr_t)vpool | (uintptr_t)out) & 15)
    return fail(RPKV_ERR_INVALID_ARG, "q, pools and out must be 16-byte aligned");
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(RPKV_ERR_INVALID_ARG, "scale must be finite and positive");
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev != p->device)
    return fail(RPKV_ERR_INVALID_ARG, "attend on a device other than the plan's");
  rpkv::AttnArgs a{};
  a.q = q;
  a.kpool = kpool;
  a.vpool = vpool;
  a.out = out;
  a.page_table = p->page_table;
  a.pt_stride = p->pt_stride;
  a.toklist = (const int32_t *)(p->dmeta + p->lay.off_tok);
  a.tok_pbase = (const int32_t *)(p->dmeta + p->lay.off_pbase);
  a.o_part = p->o_part;
  a.lse_part = p->lse_part;
  a.Hq = p->s.Hq;
  a.Hkv = p->s.Hkv;
  a.G = p->s.G();
  a.D = p->s.D;
  a.log2P = p->s.log2P;
  a.num_pages = p->s.num_pages;
  a.scale_log2 = scale * 1.4426950408889634f;
  rpkv::AttnArgs pre = a, dec = a;
  pre.items = (const Item *)(p->dmeta + p->lay.off_pre);
  pre.n_items = (int32_t)hp.prefill.size();
  dec.items = (const Item *)(p->dmeta + p->lay.off_dec);
  dec.n_items = (int32_t)hp.decode.size();
  rpkv_status st = RPKV_OK;
  if (p->s.dtype == RPKV_BF16) {
    if (pre.n_items > 0 && dec.n_items > 0)
      st = timed(p, RPKV_KERNEL_FUSED, stream,
                 [&] { return rpkv::launch_fused_bf16(pre, dec, hp.tiles_per_block, stream); }, "fused launch");
    else if (pre.n_items > 0)
      st = timed(p, RPKV_KERNEL_PREFILL, stream, [&] { return rpkv::launch_prefill_bf16(pre, hp.tiles_per_block, stream); },
                 "prefill launch");
    else if (dec.n_items > 0)
      st = timed(p, RPKV_KERNEL_DECODE, stream, [&] { return rpkv::launch_decode_bf16(dec, stream); },
                 "decode launch");
  } else {
    if (pre.n_items > 0)
      st = timed(p, RPKV_KERNEL_F32, stream, [&] { return rpkv::launch_attn_f32(pre, stream); },
                 "fp32 launch");
    if (st == RPKV_OK && dec.n_items > 0)
      st = timed(p, RPKV_KERNEL_F32, stream, [&] { return rpkv::launch_attn_f32(dec, stream); },
                 "fp32 launch");
  }
  if (st == RPKV_OK && !hp.merge.empty()) {
    const int32_t *mg = (const int32_t *)(p->dmeta + p->lay.off_merge);
    st = timed(p, RPKV_KERNEL_MERGE, stream, [&] {
      return rpkv::launch_merge(mg, (int32_t)(hp.merge.size() / 3), p->o_part, p->lse_part, out,
                                p->s.Hq, p->s.D, p->s.dtype, stream);
    }, "merge launch");
  }
  return st;
}

rpkv_status rpkv_forward(rpkv_plan *p, const void *q, const void *k, const void *v,
                         const int32_t *slots, void *kpool, void *vpool, void *out, float scale,
                         void *stream) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (!p->prepared) return fail(RPKV_ERR_NOT_PREPARED, "forward before a successful prepare_metadata");
  if (p->hp.T > 0 && (!q || !out))
    return fail(RPKV_ERR_INVALID_ARG, "q and out must be non-NULL");
  rpkv_status st = rpkv_store_kv(p, k, v, slots, p->hp.T, kpool, vpool, stream);
  if (st != RPKV_OK) return st;
  return rpkv_attend(p, q, kpool, vpool, out, scale, stream);
}

rpkv_status rpkv_graph_decode_init(rpkv_plan *p, int32_t max_batch, int32_t q_len,
                                   int32_t max_seq_len) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (p->s.dtype != RPKV_BF16) return fail(RPKV_ERR_UNSUPPORTED, "graph decode is bf16 only");
  if (max_batch < 1 || q_len < 1 || max_seq_len < q_len)
    return fail(RPKV_ERR_INVALID_ARG, "need max_batch >= 1, q_len >= 1, max_seq_len >= q_len");
  if ((int64_t)q_len * p->s.G() > rpkv::kDecodeRows)
    return fail(RPKV_ERR_UNSUPPORTED, "q_len * Hq / Hkv must be <= 16 (one split-KV item)");
  if ((int64_t)max_seq_len > (int64_t)p->s.max_pages_per_req * p->s.P)
    return fail(RPKV_ERR_CAPACITY, "max_seq_len exceeds max_pages_per_req * page_size");
  if ((int64_t)max_batch * q_len > INT32_MAX / 32)
    return fail(RPKV_ERR_INVALID_ARG, "max_batch * q_len too large");
  int32_t chunk = 0, maxc = 0;
  rpkv::graph_decode_chunks(max_batch, p->s.Hkv, max_seq_len, &chunk, &maxc);
  int dev = 0;
  int e = hipGetDevice(&dev);
  if (e) return hip_fail(e, "hipGetDevice");
  const size_t rows = (size_t)max_batch * q_len * maxc * p->s.Hq;
  const size_t obytes = align256(rows * p->s.D * sizeof(float));
  const size_t bytes = obytes + align256(rows * sizeof(float));
  if (p->g_opart) {
    e = hipDeviceSynchronize();
    if (e) return hip_fail(e, "hipDeviceSynchronize");
    (void)hipFree(p->g_opart);
    p->g_opart = p->g_lse = nullptr;
    p->g_max_batch = 0;
  }
  void *buf = nullptr;
  e = hipMalloc(&buf, bytes);
  if (e) return hip_fail(e, "hipMalloc (graph decode partials)");
  p->g_opart = (float *)buf;
  p->g_lse = (float *)((char *)buf + obytes);
  p->g_max_batch = max_batch;
  p->g_q_len = q_len;
  p->g_chunk = chunk;
  p->g_maxc = maxc;
  p->g_max_seq = max_seq_len;
  p->g_device = dev;
  return RPKV_OK;
}

rpkv_status rpkv_graph_decode_forward(rpkv_plan *p, int32_t batch, const void *q, const void *k,
                                      const void *v, const int32_t *slot_mapping, void *kpool,
                                      void *vpool, const int32_t *seq_lens,
                                      const int32_t *page_table, int64_t pt_stride,
                                      int32_t pt_cols, void *out, float scale, void *stream) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (!p->g_opart) return fail(RPKV_ERR_NOT_PREPARED, "graph decode not initialised");
  if (batch < 0 || batch > p->g_max_batch)
    return fail(RPKV_ERR_CAPACITY, "batch exceeds the graph decode capacity");
  if (batch == 0) return RPKV_OK;
  if (!q || !k || !v || !slot_mapping || !kpool || !vpool || !seq_lens || !page_table || !out)
    return fail(RPKV_ERR_INVALID_ARG, "q, k, v, slot_mapping, pools, seq_lens, page_table, out must be non-NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)kpool | (uintptr_t)vpool |
       (uintptr_t)out) & 15)
    return fail(RPKV_ERR_INVALID_ARG, "q, k, v, pools and out must be 16-byte aligned");
  if (pt_cols < 0 || pt_stride < pt_cols ||
      (int64_t)pt_cols * p->s.P < (int64_t)p->g_max_seq)
    return fail(RPKV_ERR_INVALID_ARG, "page table must have ceil(max_seq_len / page_size) columns");
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(RPKV_ERR_INVALID_ARG, "scale must be finite and positive");
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev != p->g_device)
    return fail(RPKV_ERR_INVALID_ARG, "graph decode on a device other than its init's");
  const int32_t T = batch * p->g_q_len;
  const int64_t row_bytes = (int64_t)p->s.Hkv * p->s.D * 2;
  const int64_t num_slots = p->s.num_pages * p->s.P;
  rpkv_status st = timed(p, RPKV_KERNEL_STORE, stream, [&] {
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
  a.pstride = p->g_maxc;
  a.o_part = p->g_opart;
  a.lse_part = p->g_lse;
  a.Hq = p->s.Hq;
  a.Hkv = p->s.Hkv;
  a.G = p->s.G();
  a.D = p->s.D;
  a.log2P = p->s.log2P;
  a.num_pages = p->s.num_pages;
  a.scale_log2 = scale * 1.4426950408889634f;
  st = timed(p, RPKV_KERNEL_DECODE, stream, [&] {
    return rpkv::launch_graph_decode_bf16(a, seq_lens, p->g_q_len, p->g_chunk, p->g_maxc,
                                          p->g_max_seq, batch, stream);
  }, "graph decode launch");
  if (st != RPKV_OK || p->g_maxc <= 1) return st;
  return timed(p, RPKV_KERNEL_MERGE, stream, [&] {
    return rpkv::launch_graph_merge(seq_lens, p->g_q_len, p->g_chunk, p->g_maxc, p->g_max_seq, T,
                                    p->g_opart, p->g_lse, out, p->s.Hq, p->s.D, p->s.dtype,
                                    stream);
  }, "graph merge launch");
}

rpkv_status rpkv_build_metadata(int32_t batch, const int32_t *num_computed, const int32_t *n,
                                const uint8_t *need_logits, const int32_t *block_tables,
                                int64_t bt_stride, int32_t bt_cols, int32_t page_size,
                                int64_t max_tokens, int32_t *query_start_loc, int32_t *seq_lens,
                                int32_t *positions, int32_t *slot_mapping,
                                int32_t *logits_indices, int32_t *counts, void *stream) {
  if (batch < 0) return fail(RPKV_ERR_INVALID_ARG, "batch < 0");
  if (max_tokens < 0) return fail(RPKV_ERR_INVALID_ARG, "max_tokens < 0");
  if (page_size < 1 || page_size > 1024 || (page_size & (page_size - 1)))
    return fail(RPKV_ERR_INVALID_ARG, "page_size must be a power of two in [1, 1024]");
  if (bt_cols < 0 || bt_stride < bt_cols)
    return fail(RPKV_ERR_INVALID_ARG, "block table: need 0 <= cols <= stride");
  if (!query_start_loc || !seq_lens || !logits_indices || !counts)
    return fail(RPKV_ERR_INVALID_ARG, "query_start_loc, seq_lens, logits_indices, counts must be non-NULL");
  if (batch > 0 && (!num_computed || !n || !block_tables))
    return fail(RPKV_ERR_INVALID_ARG, "num_computed, n and block_tables must be non-NULL");
  if (max_tokens > 0 && (!positions || !slot_mapping))
    return fail(RPKV_ERR_INVALID_ARG, "positions and slot_mapping must be non-NULL");
  int log2P = 0;
  while ((1 << log2P) < page_size) ++log2P;
  const int e = rpkv::launch_build_metadata(batch, num_computed, n, need_logits, block_tables,
                                            bt_stride, bt_cols, log2P, max_tokens, query_start_loc,
                                            seq_lens, positions, slot_mapping, logits_indices,
                                            counts, stream);
  if (e) return hip_fail(e, "build_metadata launch");
  return RPKV_OK;
}

rpkv_status rpkv_timing_enable(rpkv_plan *p, int32_t enable, int32_t max_launches) {
  if (!p) return fail(RPKV_ERR_INVALID_ARG, "plan is NULL");
  if (enable && max_launches <= 0) return fail(RPKV_ERR_INVALID_ARG, "max_launches must be > 0");
  p->timing = enable != 0;
  if (!enable) return RPKV_OK;
  while ((int32_t)p->ev.size() < 2 * max_launches) {
    hipEvent_t e;
    int err = hipEventCreate(&e);
    if (err) return hip_fail(err, "hipEventCreate");
    p->ev.push_back(e);
  }
  p->max_launches = max_launches;
  p->ev_kind.assign(max_launches, 0);
  p->n_rec = 0;
  return RPKV_OK;
}

rpkv_status rpkv_timing_collect(rpkv_plan *p, rpkv_kernel_times *out) {
  if (!p || !out) return fail(RPKV_ERR_INVALID_ARG, "plan or out is NULL");
  for (int32_t i = 0; i < p->n_rec; ++i) {
    int e = hipEventSynchronize(p->ev[2 * i + 1]);
    if (e) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, p->ev[2 * i], p->ev[2 * i + 1]);
    if (e) return hip_fail(e, "hipEventElapsedTime");
    out->launches[p->ev_kind[i]] += 1;
    out->total_ms[p->ev_kind[i]] += ms;
  }
  p->n_rec = 0;
  return RPKV_OK;
}

}  // extern "C"
