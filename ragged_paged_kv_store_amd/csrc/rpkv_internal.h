// Internal declarations shared by the planner, the launcher and the kernels.
// Not part of the ABI (the ABI is include/rpkv.h).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "rpkv.h"

namespace rpkv {

// One unit of attention work.  For the MFMA prefill kernel an item is one
// workgroup (a tile of up to kPrefillRows query rows x one KV head); for the
// split-KV decode kernel an item is one wavefront (up to 16 rows); for the fp32
// kernel one workgroup of up to kF32Rows rows.  Rows are (token, head-in-group)
// pairs, token-major: row m -> token tok0 + m / G, query head kvh*G + m % G.
struct Item {
  int32_t req;   // request index: its page-table row is read
  int32_t kvh;   // KV head
  int32_t tok0;  // first packed token, or offset into the cascade token list
  int32_t ntok;  // low 16 bits: tokens the tile touches (0 = padding item,
                 // skipped); bits 16..23: rows of the first token that precede
                 // the tile (see item_rows)
  int32_t pos0;  // absolute position of tok0's query; -1 marks a cascade prefix
                 // tile (tokens from the list, every key in range visible)
  int32_t kbeg;  // keys [kbeg, kend) of the request are attended
  int32_t kend;
  int32_t split; // -1: write the final output; >= 0: write partial number
                 // `split` of each token (partial index tok_pbase[t] + split)
};
static_assert(sizeof(Item) == 32, "Item is 8 int32");

// The rows of an item are a run of the (token, head-in-group) rows of its
// tokens, token-major: run row j is token tok0 + j / G, query head kvh*G + j % G.
// A tile starts `item_row0` rows into the run (0 unless the tile was cut at a
// multiple of 128 rows inside a token, for G not dividing 128) and holds the
// rest of the run up to `cap` rows.
#if defined(__HIP__)
#define RPKV_HD __attribute__((host, device, always_inline)) inline
#else
#define RPKV_HD inline
#endif
RPKV_HD int32_t item_ntok(const Item &it) { return it.ntok & 0xffff; }
RPKV_HD int32_t item_row0(const Item &it) { return (it.ntok >> 16) & 0xff; }
RPKV_HD int32_t item_rows(const Item &it, int32_t G, int32_t cap) {
  const int32_t r = item_ntok(it) * G - item_row0(it);
  return r < cap ? r : cap;
}
RPKV_HD int32_t pack_ntok(int32_t ntok, int32_t row0) { return ntok | (row0 << 16); }
#undef RPKV_HD

constexpr int kPrefillRows = 128;     // bf16 MFMA tile: 4 waves x 32 rows
constexpr int kPrefillKeys = 64;      // keys per LDS tile
constexpr int kDecodeRows = 16;       // bf16 split-KV item: 16 MFMA columns
constexpr int kDecodeKeys = 32;       // keys per decode step
constexpr int kDecodeWavesPerBlock = 4;
// MFMA tiles per workgroup when the shape leaves it to the planner: pairs
// (8 wavefronts in ping-pong, prefill_pair.h) when the batch's tiles average at
// least this many 64-key steps; shorter tiles run one per 4-wavefront
// workgroup (prefill_tile.h), two workgroups per CU, which hides their
// fixed per-tile cost better.
constexpr int kPairMinSteps = 24;
constexpr int kF32Rows = 16;          // fp32 tile rows
constexpr int kF32Keys = 32;          // fp32 keys per LDS tile
constexpr int kNumXcd = 8;            // MI355X: 8 XCDs, blocks go round-robin
constexpr int kPrefillSlots = 512;    // MI355X: 256 CUs x 2 resident prefill tiles
// deepest nesting of shared-prefix levels the planner keeps (the keys of deeper
// levels are read by their members as part of the level above or their tails)
constexpr int kMaxCascadeDepth = 16;
// In a mixed launch a split-KV chunk is sized to the tiles' critical path:
// this many keys per 64-key tile step of it.  (A chunk streams ~20 keys/us
// beside tiles that take ~2 us per step, so 8 ends the chunks at about a third
// of the critical path, freeing their slots for the last tiles; measured
// against 4-32: C2's launch -6.7% and radix -9.3% against 24, with the merge
// included -3.4% and -6.3%; C4 and C5 unchanged; below 8 the merge grows.)
constexpr int kConcurrentKeysPerStep = 8;

// One level of the shared-prefix tree.  Its members attend the keys between the
// parent level's prefix (0 at the top) and `prefix` once, stacked together in
// MFMA tiles over the first member's page-table row; the keys past the deepest
// level a member belongs to are its own tail.
struct CascNode {
  int32_t parent;  // index of the enclosing level, -1 at the top
  int32_t prefix;  // shared keys [0, prefix), a multiple of the page size
  std::vector<int32_t> members;  // request indices, >= 2
};

// Work buffers of the planner, kept with a plan so their capacity carries over
// from batch to batch (a fresh multi-hundred-KB vector per batch costs page
// faults on every plan).
struct PlanScratch {
  std::vector<Item> tiles, pre, dec, dlast;
  std::vector<int64_t> tile_key, pre_key, work, ukey;
  std::vector<int32_t> nsplit, deepest, runs, order, idx, first, second;
};

struct HostPlan {
  int32_t batch = 0, T = 0, max_q = 0, max_k = 0;
  std::vector<int32_t> cu_q, L;
  std::vector<int32_t> csr_indptr;  // [batch+1] when the page table came in CSR form
  std::vector<Item> prefill;   // XCD-interleaved, padded to a multiple of 8
  std::vector<Item> decode;    // longest first
  std::vector<int32_t> tok_pbase;  // [T] partial base or -1
  std::vector<int32_t> merge;      // [M][3] token, partial base, count
  std::vector<int32_t> toklist;    // cascade token lists
  std::vector<CascNode> tree;      // shared-prefix levels, parents first
  int32_t cascade_depth = 0;
  int64_t n_partials = 0;
  int32_t n_cascade_items = 0, cascade_members = 0, decode_chunk = 0;
  int32_t tiles_per_block = 1;     // MFMA tiles per workgroup (1 or 2)
  int32_t n_prefill_real = 0;      // items before padding
  double plan_us = 0;
  PlanScratch tmp;
  // empty the plan, keeping every vector's capacity
  void reset() {
    batch = T = max_q = max_k = 0;
    cu_q.clear(); L.clear(); csr_indptr.clear(); prefill.clear(); decode.clear();
    tok_pbase.clear(); merge.clear(); toklist.clear(); tree.clear();
    cascade_depth = 0;
    n_partials = 0;
    n_cascade_items = cascade_members = decode_chunk = 0;
    n_prefill_real = 0;
    tiles_per_block = 1;
    plan_us = 0;
  }
};

struct Shape {
  int32_t Hq, Hkv, D, P, log2P, dtype, max_batch, max_pages_per_req;
  int64_t num_pages, max_tokens;
  int32_t decode_max_rows, split_target, split_min_keys, prefix_detect_keys;
  int32_t tiles_per_block;  // 0: chosen per batch
  int32_t check_slots;      // debug: store_kv validates slot_mapping on the host
  int32_t G() const { return Hq / Hkv; }
};

// Entries of each array of the work partition's device copy.  meta_caps gives
// the most any batch within a shape's capacities can need (the plan's device
// buffers are sized from it once); meta_counts what one planned batch needs.
struct MetaCounts {
  int64_t pre, dec, pbase, merge, tok, indptr;
};
struct MetaLayout {
  size_t off_pre, off_dec, off_pbase, off_merge, off_tok, off_indptr, bytes;
};
MetaCounts meta_caps(const Shape &s);
MetaCounts meta_counts(const HostPlan &p, int32_t max_batch);
MetaLayout meta_layout(const MetaCounts &c);

// Validate a slot_mapping on the host: every non-negative slot below num_slots
// and distinct.  Returns the first offending token or -1; `scratch` is reused.
int64_t find_bad_slot(const int32_t *slots, int64_t n, int64_t num_slots,
                      std::vector<int64_t> *scratch, std::string *msg);

// Key chunk of the graph-capturable decode for batches of up to max_batch
// requests with lengths up to max_seq: chunks per request enough that a full
// batch gives about 4 wavefronts per resident slot (2048 on the chip), between 2
// and 32 (the merge's one-round-trip path); chunks of >= 256 keys, a multiple
// of 64.  *maxc = ceil(max_seq / chunk).
void graph_decode_chunks(int64_t max_batch, int32_t Hkv, int32_t max_seq, int32_t *chunk,
                         int32_t *maxc);

// Validate a shape; on failure returns the status and fills msg.
rpkv_status check_shape(const rpkv_shape *s, Shape *out, std::string *msg);

// Build the work partition of one batch on the host into *out (emptied first,
// its vectors' capacity reused; its contents are unspecified after an error).
rpkv_status plan_batch_host(const Shape &s, int32_t batch, const int32_t *cu,
                            const int32_t *L, int32_t cols, const int32_t *pt_host,
                            const rpkv_prefix_group *groups, int32_t ngroups, HostPlan *out,
                            std::string *msg);

// Kernel launchers (defined in the .hip files).  All enqueue on `stream`.
struct AttnArgs {
  const void *q;
  const void *kpool;
  const void *vpool;
  void *out;
  const int32_t *page_table;
  int64_t pt_stride;
  const Item *items;
  int32_t n_items;
  const int32_t *toklist;
  const int32_t *tok_pbase;
  float *o_part;      // [partials, Hq, D]
  float *lse_part;    // [partials, Hq] (base-2 log-sum-exp of scaled logits)
  int32_t Hq, Hkv, G, D, log2P;
  int64_t num_pages;
  float scale_log2;   // scale * log2(e)
  int32_t pstride;    // partials per token when tok_pbase is NULL (graph decode)
};

int launch_store_kv(const void *k, const void *v, const int32_t *slots, int64_t T,
                    int64_t row_bytes, int64_t num_slots, void *kpool, void *vpool,
                    void *stream);
int launch_prefill_bf16(const AttnArgs &a, int tiles_per_block, void *stream);
int launch_decode_bf16(const AttnArgs &a, void *stream);
// split-KV chunks and MFMA tiles in one grid (chunks first)
int launch_fused_bf16(const AttnArgs &pre, const AttnArgs &dec, int tiles_per_block, void *stream);
int launch_attn_f32(const AttnArgs &a, void *stream);
int launch_graph_decode_bf16(const AttnArgs &a, const int32_t *seq_lens, int32_t q_len,
                             int32_t chunk, int32_t maxc, int32_t max_seq, int32_t batch,
                             void *stream);
int launch_graph_merge(const int32_t *seq_lens, int32_t q_len, int32_t chunk, int32_t maxc,
                       int32_t max_seq, int32_t T, const float *o_part, const float *lse_part, void *out,
                       int32_t Hq, int32_t D, int32_t dtype, void *stream);
int launch_csr_to_dense(int32_t B, const int32_t *indptr, const int32_t *indices, int32_t *dense,
                        int64_t stride, void *stream);
int launch_rewrite_blocks(int32_t B, const int32_t *table, int64_t stride, int32_t cols,
                          int32_t factor, int32_t *out, int64_t out_stride, void *stream);
int launch_build_metadata(int32_t B, const int32_t *nc, const int32_t *n, const uint8_t *need,
                          const int32_t *tables, int64_t stride, int32_t cols, int32_t log2P,
                          int64_t max_tokens, int32_t *qsl, int32_t *seq, int32_t *positions,
                          int32_t *slots, int32_t *lg, int32_t *counts, void *stream);
int launch_merge(const int32_t *merge, int32_t n_merge, const float *o_part,
                 const float *lse_part, void *out, int32_t Hq, int32_t D, int32_t dtype,
                 void *stream);

}  // namespace rpkv
