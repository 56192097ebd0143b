// The plan object behind the C ABI's opaque rpkv_plan, and helpers shared by
// the ABI's source files.  Not part of the ABI (the ABI is include/rpkv.h).
#pragma once

#include <hip/hip_runtime_api.h>

#include <string>
#include <vector>

#include "rpkv_internal.h"

struct rpkv_plan {
  rpkv::Shape s{};
  rpkv::HostPlan hp;
  rpkv::HostPlan hp_next;  // planned into, then swapped with hp when the batch is valid
  bool planned = false;
  bool prepared = false;
  int device = -1;
  // device copy of the work partition, sized once for the shape's capacities
  // (rpkv::meta_caps) at the first prepare; every batch's copy fits in it
  char *dmeta = nullptr;
  size_t meta_cap = 0;        // bytes of dmeta and of each staging buffer
  rpkv::MetaLayout lay{};     // the planned batch's layout
  int64_t n_alloc = 0;        // allocations made by ensure_device
  // dense copy of a CSR page table (plan-owned, [max_batch, max_pages_per_req])
  int32_t *csr_table = nullptr;
  // pinned staging, two buffers so a new batch never overwrites one in flight
  char *hmeta[2] = {nullptr, nullptr};
  hipEvent_t hev[2] = {nullptr, nullptr};
  bool hev_live[2] = {false, false};
  int hcur = 0;
  // bound per batch
  const int32_t *page_table = nullptr;
  int64_t pt_stride = 0;
  float *o_part = nullptr;
  float *lse_part = nullptr;
  size_t ws_need = 0;
  // timing
  bool timing = false;
  int32_t max_launches = 0;
  std::vector<hipEvent_t> ev;
  std::vector<int32_t> ev_kind;
  int32_t n_rec = 0;
  // host copy of a slot_mapping for the check_slots debug mode
  std::vector<int32_t> slots_host;
  std::vector<int64_t> slots_key;
  // graph-capturable decode: fixed capacities and plan-owned partials
  int32_t g_max_batch = 0, g_q_len = 0, g_chunk = 0, g_maxc = 0, g_max_seq = 0;
  float *g_opart = nullptr;
  float *g_lse = nullptr;
  int g_device = -1;
};

namespace rpkv {

// Record the calling thread's error message (rpkv_last_error) and return st.
rpkv_status fail(rpkv_status st, const std::string &msg);
// An RPKV_ERR_HIP status naming the HIP call and the runtime's message.
rpkv_status hip_fail(int err, const char *what);

// Run one launch; with timing enabled, HIP events are recorded on the launch
// stream around it (rpkv_timing_collect adds up their durations by kind).
template <class F>
inline rpkv_status timed(rpkv_plan *p, int kind, void *stream, F &&launch, const char *what) {
  const bool rec = p->timing && p->n_rec < p->max_launches;
  if (rec) {
    int e = hipEventRecord(p->ev[2 * p->n_rec], (hipStream_t)stream);
    if (e) return hip_fail(e, "hipEventRecord");
  }
  int err = launch();
  if (err) return hip_fail(err, what);
  if (rec) {
    int e = hipEventRecord(p->ev[2 * p->n_rec + 1], (hipStream_t)stream);
    if (e) return hip_fail(e, "hipEventRecord");
    p->ev_kind[p->n_rec++] = kind;
  }
  return RPKV_OK;
}

}  // namespace rpkv
