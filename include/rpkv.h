/*
 * rpkv.h -- C ABI of the ragged, paged KV-store attention library for MI355X
 * (gfx950).  One step of one attention layer over a packed batch that mixes
 * prefill, chunked-prefill and decode requests:
 *
 *   1. store_kv: this step's new K/V rows are scattered into the layer's paged
 *      KV pool by slot;
 *   2. attend:   the queries of request i, rows [cu_q[i], cu_q[i+1]) of the
 *      packed q, attend to the first cache_seqlens[i] pool slots named by row i
 *      of the page table, with a bottom-right causal mask and grouped KV heads.
 *
 * Sources (page title, then section):
 *  - mini-sglang "The attention backend and a reference implementation",
 *    "The interface": metadata is prepared once per batch and reused by every
 *    layer; forward(q, k, v, layer) writes the new K/V before reading the pool.
 *    "Variable-length, paged attention with prefixes": cu_seqlens_q,
 *    cache_seqlens, page-table rows, the bottom-right mask (query r of n with L
 *    keys sits at position L-n+r and sees keys 0..L-n+r), GQA head sharing.
 *  - vLLM "Attention backends: backend, metadata builder and implementation",
 *    Step 2: the implementation writes into a caller-provided output; the KV
 *    cache update can be a separate call that scatters by slot_mapping.
 *    Step 1: a backend answers capability questions (head sizes, dtypes).
 *  - SGLang source walkthrough "Attention backends", 3.1 (plan once, then run;
 *    a caller-provided device workspace), 3.2 (the page table in CSR form; the
 *    radix cache fills it, so reused prefixes carry the same page ids), 3.3
 *    (cascade: a shared prefix attended once and merged with each request's own
 *    tail by log-sum-exp; the multi-level form takes one level per depth of the
 *    radix tree), 6 (a mixed batch is split by token into decode work and
 *    prefill work).
 *  - "Variable-length batching and one mixed forward pass", exercise 2: pure
 *    decode work uses split-KV (flash-decoding) kernels; "Source code": the
 *    logits indices are cu_q[1:] - 1.
 *
 * Conventions for every call
 *  - Device pointers are HIP device memory on the current device; host pointers
 *    are ordinary host memory.  The library never frees caller memory.
 *  - A stream argument is a hipStream_t passed as void* (NULL = default stream).
 *    All device work of a call is enqueued on that stream; no call blocks on the
 *    device except where stated.  Calls are not thread-safe on one plan.
 *  - Every call returns an rpkv_status.  On failure nothing is enqueued, no
 *    caller memory is written, and rpkv_last_error() describes the reason.
 *  - Layouts (row-major, contiguous):
 *      q, out          [T, Hq, D]                    T = cu_q[batch]
 *      k, v (new rows) [T, Hkv, D]
 *      K pool, V pool  [num_pages, page_size, Hkv, D] for one layer, i.e.
 *                      [num_slots, Hkv, D] with slot = page * page_size + offset
 *      page table      [batch, >= cols] int32 page ids, row stride in elements;
 *                      logical position x of request i lives in slot
 *                      table[i][x / page_size] * page_size + x % page_size.
 *    Entries beyond a row's first ceil(L/page_size) are never read.
 *  - Query head h reads KV head h / (Hq / Hkv).
 */
#ifndef RPKV_H
#define RPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rpkv_status {
  RPKV_OK = 0,
  RPKV_ERR_INVALID_ARG = 1,         /* an argument breaks a documented rule       */
  RPKV_ERR_UNSUPPORTED = 2,         /* no kernel for this head size/dtype/page    */
  RPKV_ERR_WORKSPACE_TOO_SMALL = 3, /* see rpkv_workspace_bytes                    */
  RPKV_ERR_NOT_PREPARED = 4,        /* attend/forward before a successful prepare  */
  RPKV_ERR_HIP = 5,                 /* the HIP runtime reported an error           */
  RPKV_ERR_CAPACITY = 6             /* batch exceeds the plan's stated capacities  */
} rpkv_status;

typedef enum rpkv_dtype {
  RPKV_BF16 = 0, /* bfloat16 in, fp32 accumulate and softmax, bf16 out (RNE) */
  RPKV_F32 = 1   /* float32 throughout                                       */
} rpkv_dtype;

/* Fixed properties of one attention layer type and the plan's capacities.
 * Zero in a tuning field selects the library default. */
typedef struct rpkv_shape {
  int32_t num_q_heads;       /* Hq                                              */
  int32_t num_kv_heads;      /* Hkv; Hq % Hkv == 0; Hq / Hkv <= 128 (bf16) or
                                <= 16 (f32)                                     */
  int32_t head_dim;          /* D: 128 (bf16); 64 or 128 (f32)                  */
  int32_t page_size;         /* tokens per page: a power of two in [1, 1024]    */
  int32_t dtype;             /* rpkv_dtype of q, k, v, the pools and out        */
  int32_t max_batch;         /* capacity: requests per batch                    */
  int64_t num_pages;         /* pages in one layer's pool                       */
  int64_t max_tokens;        /* capacity: new tokens per batch (T)              */
  int32_t max_pages_per_req; /* capacity: page-table columns a request may use  */
  int32_t decode_max_rows;   /* tuning: a request is decode-type iff
                                n*Hq/Hkv <= this (default 16, at most 16)      */
  int32_t split_target;      /* tuning: target number of decode work items per
                                launch when choosing split-KV chunks (default
                                3072)                                           */
  int32_t split_min_keys;    /* tuning: smallest split-KV chunk in keys
                                (default 64; rounded up to 32)                  */
  int32_t prefix_detect_keys;/* cascade: when > 0, a batch planned with a host
                                page table and no cascade hints gets its
                                shared-prefix tree from the page-table rows;
                                a level is kept only if it adds at least this
                                many keys to its parent level (0: off)          */
  int32_t tiles_per_block;   /* tuning: MFMA tiles per workgroup: 1 (four
                                wavefronts, one tile), 2 (eight wavefronts, two
                                tiles in ping-pong), 0 (default): 2 when the
                                batch's tiles average at least 24 key steps of
                                64 and pages hold >= 16 keys, else 1            */
  int32_t check_slots;       /* debug: when nonzero, rpkv_store_kv and
                                rpkv_forward copy slot_mapping to the host
                                (blocking the host on the stream) and reject
                                duplicate or out-of-range slots before
                                enqueueing anything (0: off)                    */
} rpkv_shape;

/* Cascade hint (SGLang source walkthrough "Attention backends", 3.3 "Cascade
 * Inference": a shared prefix is attended once and merged with each request's
 * own part by log-sum-exp; the multi-level form takes one level per depth of the
 * radix tree).  Requests [first_req, first_req + num_reqs) of the batch have
 * identical page ids in their first prefix_len / page_size columns (prefix_len a
 * multiple of page_size; 0 makes the hint a no-op).  The shared prefix is read
 * once for all eligible members and merged with each member's own tail.  A member
 * is eligible if it is decode-type and none of its new tokens lies in the prefix
 * (L - n >= prefix_len); other members are computed without the cascade.
 * Hints may nest to form several levels: a hint whose range lies inside another's
 * must have a longer prefix, and its members then attend only the keys between
 * the two prefixes at that level.  Ranges that overlap without nesting are an
 * error.  A level with fewer than two eligible members is skipped (its nested
 * levels attach to the next level up). */
typedef struct rpkv_prefix_group {
  int32_t first_req;
  int32_t num_reqs;
  int32_t prefix_len;
} rpkv_prefix_group;

typedef struct rpkv_plan rpkv_plan;

/* What the last successful plan holds (host-side summary). */
typedef struct rpkv_plan_info {
  int32_t batch;
  int32_t num_tokens;          /* T                                       */
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int32_t num_prefill_items;   /* MFMA tiles, incl. cascade prefix tiles  */
  int32_t num_decode_items;    /* split-KV chunks (one wave each)         */
  int32_t num_cascade_items;   /* of which shared-prefix level tiles      */
  int32_t num_merge_tokens;    /* tokens whose heads are merged           */
  int64_t num_partials;        /* partial results (token x split)         */
  int64_t workspace_bytes;     /* device workspace the batch needs        */
  int32_t decode_chunk;        /* split-KV chunk in keys                  */
  int32_t cascade_members;     /* requests served through the cascade     */
  double plan_host_us;         /* host time of the last plan              */
  int32_t num_cascade_levels;  /* shared-prefix levels (tree nodes)       */
  int32_t cascade_depth;       /* longest chain of nested levels          */
  int32_t num_cascade_level_members; /* sum of the levels' member counts  */
  int32_t tiles_per_block;     /* MFMA tiles per workgroup this batch     */
  int64_t metadata_bytes;      /* device copy of this batch's partition   */
  int64_t metadata_capacity_bytes; /* the plan's fixed metadata buffer:
                                  every batch within the capacities fits */
  int64_t buffer_allocations;  /* device and pinned allocations the plan's
                                  prepare calls have made (all at the
                                  first; graph decode's are not counted) */
} rpkv_plan_info;

/* Kernel timing (benchmarks): per kernel kind, launches and summed durations
 * measured with HIP events recorded on the launch stream around each launch. */
typedef enum rpkv_kernel_kind {
  RPKV_KERNEL_STORE = 0,
  RPKV_KERNEL_PREFILL = 1, /* bf16 MFMA tiles, incl. cascade prefix */
  RPKV_KERNEL_DECODE = 2,  /* bf16 split-KV                         */
  RPKV_KERNEL_MERGE = 3,   /* log-sum-exp merge                     */
  RPKV_KERNEL_F32 = 4,     /* fp32 tiles                            */
  RPKV_KERNEL_FUSED = 5,   /* split-KV chunks and MFMA tiles in one
                              launch (mixed bf16 batches)           */
  RPKV_KERNEL_KINDS = 6
} rpkv_kernel_kind;

typedef struct rpkv_kernel_times {
  int64_t launches[8];
  double total_ms[8];
} rpkv_kernel_times;

/* ---------------------------------------------------------------- errors */

/* Static, human-readable name of a status. */
const char *rpkv_status_string(rpkv_status status);

/* Message of the last failed call made on this thread ("" if none).  The
 * pointer stays valid until the next call on this thread. */
const char *rpkv_last_error(void);

/* ------------------------------------------------------------- plan setup */

/* Capability query (vLLM Step 1): RPKV_OK if a plan can be made for this
 * shape, else RPKV_ERR_UNSUPPORTED or RPKV_ERR_INVALID_ARG.  No device work. */
rpkv_status rpkv_supports(const rpkv_shape *shape);

/* Create a plan for one layer type (mini-sglang "The attention backend and a
 * reference implementation", "The interface": a backend is built once for the
 * model's head shape and KV pool; SGLang source walkthrough "Attention
 * backends", 3.1: fixed-size metadata buffers allocated ahead of the batches).
 * Host-only: allocates host memory and fixes the metadata capacity, an upper
 * bound of the work partition of any batch within the shape's capacities
 * (max_batch, max_tokens, max_pages_per_req; rpkv_plan_info reports it).  The
 * device buffers of that capacity (plus a [max_batch, max_pages_per_req] int32
 * table for CSR page tables) and two pinned staging buffers are allocated once
 * by the first prepare; no later prepare allocates or frees memory.  *out
 * receives the plan, owned by the library until rpkv_plan_destroy. */
rpkv_status rpkv_plan_create(const rpkv_shape *shape, rpkv_plan **out);

/* Release a plan and its device buffers (waits for the device). NULL is a no-op. */
void rpkv_plan_destroy(rpkv_plan *plan);

/* --------------------------------------------------------- once per batch */

/* Host half of prepare_metadata: validate the batch and build the work
 * partition (classification into decode-type and prefill-type requests, MFMA
 * tiles, split-KV chunks, cascade tiles, partial-result layout, merge list).
 * No device work; usable without a GPU.
 *   batch              requests, 0 <= batch <= max_batch
 *   cu_seqlens_q_host  [batch+1] host, cu[0] = 0, non-decreasing, cu[batch] <=
 *                      max_tokens; n_i = cu[i+1]-cu[i]
 *   cache_seqlens_host [batch] host, L_i >= n_i (KV length including this step)
 *   page_table_cols    columns readable in each page-table row; needs
 *                      ceil(L_i / page_size) <= cols <= max_pages_per_req
 *   page_table_host    optional host copy [batch, cols] (row stride = cols); when
 *                      given, page ids are checked to be in [0, num_pages) and
 *                      cascade hints are checked against it; with no hints and
 *                      shape.prefix_detect_keys > 0 the shared-prefix levels
 *                      are found from it (radix tree of the eligible requests'
 *                      page ids over their pages cached before this step)
 *   groups_host        optional cascade hints [num_groups], possibly nested
 * Errors: INVALID_ARG (rule broken), CAPACITY (capacities exceeded). */
rpkv_status rpkv_plan_batch(rpkv_plan *plan, int32_t batch, const int32_t *cu_seqlens_q_host,
                            const int32_t *cache_seqlens_host, int32_t page_table_cols,
                            const int32_t *page_table_host, const rpkv_prefix_group *groups_host,
                            int32_t num_groups);

/* prepare_metadata (once per batch, reused by every layer): rpkv_plan_batch,
 * then one asynchronous host-to-device copy of the work partition on `stream`.
 *   page_table_dev     device [batch, stride] int32; must stay valid and
 *                      unchanged while attend/forward of this batch run
 *   page_table_stride  elements between rows (>= page_table_cols)
 *   workspace_dev      caller-owned device scratch for split-KV / cascade
 *                      partials, 256-byte aligned; may be NULL when the batch
 *                      needs none.  If it is smaller than the batch needs, the
 *                      call fails with WORKSPACE_TOO_SMALL and
 *                      rpkv_workspace_bytes reports the size to provide.
 * The host arrays may be reused by the caller as soon as the call returns.
 * Page ids outside [0, num_pages) that reach a kernel are clamped (results
 * unspecified, no out-of-bounds access).
 * Streams: the work partition is uploaded on `stream` into one plan-owned
 * device buffer that every batch reuses.  This batch's attend/forward calls must
 * be ordered after this call on the device (the same stream, or one that waits
 * on it), and the next prepare on the plan must be ordered after the last of
 * them; one stream for all of a plan's calls satisfies both.  The host-side
 * staging is double-buffered: the call blocks only if the upload two batches
 * back has not finished. */
rpkv_status rpkv_prepare_metadata(rpkv_plan *plan, int32_t batch, const int32_t *cu_seqlens_q_host,
                                  const int32_t *cache_seqlens_host, const int32_t *page_table_dev,
                                  int64_t page_table_stride, int32_t page_table_cols,
                                  const int32_t *page_table_host,
                                  const rpkv_prefix_group *groups_host, int32_t num_groups,
                                  void *workspace_dev, size_t workspace_bytes, void *stream);

/* prepare_metadata with the page table in FlashInfer's CSR form ("SGLang source
 * walkthrough: Attention backends", 3.2 Page Table): request i's pages are
 * page_indices[page_indptr[i] .. page_indptr[i+1]) and its last page holds
 * last_page_len[i] tokens, so L_i = (pages_i - 1) * page_size + last_page_len[i]
 * (0 for a request without pages).  The lengths are derived on the host; the
 * rows are expanded into a plan-owned dense table on `stream` after the
 * metadata upload (attend/forward must follow on the same stream).
 *   page_indptr_host    [batch+1] host, page_indptr[0] = 0, non-decreasing,
 *                       pages_i <= max_pages_per_req
 *   last_page_len_host  [batch] host, in [1, page_size] for requests with pages
 *   page_indices_dev    device int32 [page_indptr[batch]]
 *   page_indices_host   optional host copy (page ids then checked, cascade hints
 *                       checked, shared prefixes detectable), else NULL
 * Other arguments and errors as rpkv_prepare_metadata. */
rpkv_status rpkv_prepare_metadata_csr(rpkv_plan *plan, int32_t batch,
                                      const int32_t *cu_seqlens_q_host,
                                      const int32_t *page_indptr_host,
                                      const int32_t *last_page_len_host,
                                      const int32_t *page_indices_dev,
                                      const int32_t *page_indices_host,
                                      const rpkv_prefix_group *groups_host, int32_t num_groups,
                                      void *workspace_dev, size_t workspace_bytes, void *stream);

/* Rewrite a block table whose blocks hold `factor` kernel pages each into a
 * table of kernel pages (vLLM "Attention backends", Step 5: the attention group
 * rewrites the block table when the kernel's blocks are smaller than the cache
 * manager's): out[i][j*factor + r] = table[i][j] * factor + r for j < cols,
 * r < factor.  Device int32 arrays owned by the caller, one kernel on `stream`.
 *   table [batch, stride] with cols valid columns; out [batch, out_stride],
 *   out_stride >= cols * factor. */
rpkv_status rpkv_rewrite_block_table(int32_t batch, const int32_t *table, int64_t stride,
                                     int32_t cols, int32_t factor, int32_t *out,
                                     int64_t out_stride, void *stream);

/* Device workspace bytes the last planned batch needs (0 if none). */
rpkv_status rpkv_workspace_bytes(const rpkv_plan *plan, size_t *bytes);

/* get_last_indices: out_host[i] = cu_q[i+1] - 1 for the planned batch, or -1
 * for a request with no queries.  out_host has room for `batch` entries. */
rpkv_status rpkv_last_indices(const rpkv_plan *plan, int32_t *out_host);

/* Summary of the last planned batch. */
rpkv_status rpkv_plan_get_info(const rpkv_plan *plan, rpkv_plan_info *info);

/* One-line text summary of the last planned batch, for logs (mini-sglang
 * "Creating a backend: one or a pair" logs the backend a run uses; here the
 * choice is per batch): request classes, MFMA tiles and tiles per workgroup,
 * split-KV chunks and their length, cascade levels, partials and merged tokens,
 * metadata bytes and host planning time.  Writes at most size bytes into buf,
 * always NUL-terminated (truncated if short; 512 bytes always suffice).
 * NOT_PREPARED before the first successful plan.  With the environment variable
 * RPKV_LOG_PLANS set (and not "0") when the library first plans, every
 * successful plan prints this line to stderr, prefixed "rpkv: ". */
rpkv_status rpkv_plan_summary(const rpkv_plan *plan, char *buf, size_t size);

/* Host copy of the last plan's work items for inspection: kind 0 = prefill
 * tiles, 1 = decode chunks.  Each item is 8 int32: request, KV head, first
 * token (or cascade token-list offset), token count (bits 0..15) with a row
 * offset (bits 16..23), position of the first token (-1 for a cascade prefix
 * tile), key begin, key end, split index (-1 = final output).  An item's rows
 * are its tokens' (token, head) rows in token-major order (row j: token
 * first + j / G, head KV head * G + j % G), starting at the row offset and
 * holding at most 128 rows (a bf16 tile) -- the offset is nonzero only where a
 * request's rows are cut every 128 rows for G not dividing 128.  Padding items
 * (token count 0) are included.  Writes min(capacity, count) items; *count
 * receives the total. */
rpkv_status rpkv_plan_get_items(const rpkv_plan *plan, int32_t kind, int32_t *items_host,
                                int32_t capacity, int32_t *count);

/* Host copy of the cascade token list (token ids of each cascade prefix tile,
 * addressed by the tile's token-list offset). */
rpkv_status rpkv_plan_get_token_list(const rpkv_plan *plan, int32_t *out_host, int32_t capacity,
                                     int32_t *count);

/* Host copy of the last plan's shared-prefix levels (from hints or detected),
 * parents before children.  Level k: parent_host[k] (index of the enclosing
 * level or -1), prefix_host[k] (shared keys [0, prefix)), and its member requests
 * members_host[member_indptr_host[k] .. member_indptr_host[k+1]) in ascending
 * order.  Sizes come from rpkv_plan_get_info: num_cascade_levels (arrays of
 * that many entries, member_indptr_host one more) and num_cascade_level_members.
 * Errors: CAPACITY if max_levels or max_members is too small (nothing written). */
rpkv_status rpkv_plan_get_cascade_tree(const rpkv_plan *plan, int32_t max_levels,
                                       int32_t max_members, int32_t *parent_host,
                                       int32_t *prefix_host, int32_t *member_indptr_host,
                                       int32_t *members_host);

/* ---------------------------------------------------------- once per layer */

/* store_kv / do_kv_cache_update (mini-sglang "The interface": forward writes
 * this step's K/V into the pool before attending; vLLM "Attention backends",
 * Step 2: the cache update scatters new rows by slot_mapping): for t <
 * num_tokens, K pool row slot_mapping[t] = k[t] and V pool row slot_mapping[t]
 * = v[t], bit for bit.  A negative slot is a padding token and writes nothing; a
 * slot >= num_pages*page_size is skipped (never written).  Slots must be
 * distinct: duplicates race (which row lands is unspecified).  With the shape's
 * check_slots set, duplicates and out-of-range slots are rejected with
 * INVALID_ARG before anything is enqueued (see rpkv_check_slot_mapping).  Uses
 * only the plan's shape; does not need a prepared batch.
 *   k, v          device [num_tokens, Hkv, D]
 *   slot_mapping  device int32 [num_tokens]
 *   k_pool/v_pool device [num_pages*page_size, Hkv, D] of one layer */
rpkv_status rpkv_store_kv(rpkv_plan *plan, const void *k, const void *v,
                          const int32_t *slot_mapping, int64_t num_tokens, void *k_pool,
                          void *v_pool, void *stream);

/* Host-side check of a slot_mapping (the store is a scatter by slot, vLLM
 * "Attention backends", Step 2: two tokens naming one slot race): INVALID_ARG,
 * naming the first offending token, if a slot is >= num_pages*page_size or
 * equals an earlier token's slot; negative slots (padding) are ignored.  No
 * device work; usable without a GPU.  slots_host [num_tokens] host int32. */
rpkv_status rpkv_check_slot_mapping(const rpkv_plan *plan, const int32_t *slots_host,
                                    int64_t num_tokens);

/* attend (mini-sglang "The attention backend and a reference implementation",
 * "Variable-length, paged attention with prefixes": each request's packed
 * queries attend its first cache_seqlens[i] pool slots through its page-table
 * row, bottom-right causal mask, query head h reading KV head h / (Hq / Hkv);
 * SGLang source walkthrough "Attention backends", 3.3 and 6: decode work split
 * over key chunks and shared prefixes merged by log-sum-exp):
 * out[t, h, :] = softmax over the visible keys of request i(t) of
 * scale * <q[t,h,:], K[.]> applied to V, for every token of the prepared batch.
 * Must be enqueued after this layer's store_kv (same stream order).
 *   q     device [T, Hq, D];  out device [T, Hq, D], caller-allocated, must not
 *         alias q or the pools;  scale usually 1/sqrt(D), finite and > 0. */
rpkv_status rpkv_attend(rpkv_plan *plan, const void *q, const void *k_pool, const void *v_pool,
                        void *out, float scale, void *stream);

/* forward(q, k, v, layer) (mini-sglang "The interface": one call per layer
 * that writes the step's K/V and then attends, the metadata prepared once per
 * batch): rpkv_store_kv of the batch's T tokens, then rpkv_attend, on one
 * stream (write first, then read).  The layer is chosen by the pool pointers
 * passed. */
rpkv_status rpkv_forward(rpkv_plan *plan, const void *q, const void *k, const void *v,
                         const int32_t *slot_mapping, void *k_pool, void *v_pool, void *out,
                         float scale, void *stream);

/* ---------------------------------------------- graph-capturable decode */

/* Pure-decode steps for HIP-graph capture and replay (the pages' capture
 * interface: mini-sglang "The attention backend and a reference
 * implementation", the capture methods of the backend interface; vLLM
 * "Attention backends", Step 6, support for uniform decode batches).  A uniform
 * batch: request i has q_len new tokens, rows i*q_len .. of q/k/v/out, and a
 * KV length L_i (including them) read from a device array at run time, so one
 * captured sequence of launches replays for any lengths: update seq_lens, the
 * page table, slot_mapping and q/k/v in place (rpkv_build_metadata can write
 * seq_lens and slot_mapping on the device), then replay.
 *
 * rpkv_graph_decode_init: fixes the capacities (max_batch requests, q_len new
 * tokens each, lengths up to max_seq_len), picks one key chunk (>= 256 keys; 2 to
 * 32 chunks per request, more for small batches) and allocates the plan-owned
 * partial workspace.
 * Call it outside capture.  bf16 only; q_len * Hq / Hkv <= 16. */
rpkv_status rpkv_graph_decode_init(rpkv_plan *plan, int32_t max_batch, int32_t q_len,
                                   int32_t max_seq_len);

/* rpkv_graph_decode_forward: store_kv of the batch*q_len tokens, then attention
 * of each request's rows over its L_i keys (bottom-right causal mask, split-KV
 * chunks merged by log-sum-exp), on `stream`.  No host synchronisation, no
 * allocation, grids fixed by `batch`: capturable.
 *   seq_lens    device int32 [batch]: q_len <= L_i <= max_seq_len (a request with
 *               L_i outside that range is skipped: no key is read and its
 *               output rows are not written)
 *   page_table  device int32 [batch, pt_stride], pt_cols >= ceil(max_seq_len / P)
 *               valid columns
 *   q, out      device [batch*q_len, Hq, D]; k, v [batch*q_len, Hkv, D];
 *   slot_mapping device int32 [batch*q_len] (as for rpkv_store_kv). */
rpkv_status rpkv_graph_decode_forward(rpkv_plan *plan, int32_t batch, const void *q, const void *k,
                                      const void *v, const int32_t *slot_mapping, void *k_pool,
                                      void *v_pool, const int32_t *seq_lens,
                                      const int32_t *page_table, int64_t pt_stride,
                                      int32_t pt_cols, void *out, float scale, void *stream);

/* rpkv_graph_decode_forward_noalloc: for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The step of rpkv_graph_decode_forward -- store_kv of the
 * batch*q_len tokens, then split-KV attention merged by log-sum-exp -- with no
 * rpkv_graph_decode_init and no allocation: q_len and max_seq_len are passed per
 * call, the key chunk is the one rpkv_graph_decode_init(plan, batch, q_len,
 * max_seq_len) would pick, and the split-KV partials live in a fixed 64 MiB
 * device array inside the library (one per GPU, held until the process ends).
 * Limits: bf16, q_len * Hq / Hkv <= 16, batch <= max_batch, batch * q_len <=
 * max_tokens, max_seq_len <= max_pages_per_req * page_size, and the partials,
 * batch * q_len * ceil(max_seq_len / chunk) * Hq * (D + 1) * 4 bytes (each part
 * rounded up to 256), must fit 64 MiB, else RPKV_ERR_CAPACITY and nothing is
 * enqueued.  Every call on a GPU reuses that GPU's array: calls that overlap on
 * one GPU (other streams, other threads, other plans) race; calls ordered on
 * one stream do not.  Nothing in the array needs clearing between calls (a
 * call reads only partials it wrote).  Other arguments, their layouts and the
 * length rule for seq_lens are those of rpkv_graph_decode_forward, with
 * pt_cols >= ceil(max_seq_len / page_size). */
rpkv_status rpkv_graph_decode_forward_noalloc(rpkv_plan *plan, int32_t batch, int32_t q_len,
                                              int32_t max_seq_len, const void *q, const void *k,
                                              const void *v, const int32_t *slot_mapping,
                                              void *k_pool, void *v_pool,
                                              const int32_t *seq_lens, const int32_t *page_table,
                                              int64_t pt_stride, int32_t pt_cols, void *out,
                                              float scale, void *stream);

/* ------------------------------------------------- device-side metadata */

/* Packed-batch metadata built on the device ("Variable-length batching and one
 * mixed forward pass": the batch builder of its worked example, and the
 * source-code notes on building positions, query_start_loc, slot_mapping and
 * logits_indices without a host loop).  From per-request, device-resident
 *   num_computed[i]  tokens of request i already in the cache (>= 0)
 *   n[i]             new tokens of request i this step (>= 0)
 *   need_logits[i]   nonzero if request i samples (NULL: every request)
 * it writes
 *   query_start_loc[B+1]  running sum of n (query_start_loc[0] = 0)
 *   seq_lens[B]           num_computed + n
 *   positions[t]          num_computed[i] + r for the r-th new token t of request i
 *   slot_mapping[t]       table[i][p / P] * P + p % P with p = positions[t]
 *                         (-1 if p / P >= bt_cols)
 *   logits_indices[m]     query_start_loc[i+1] - 1 for the m-th request (in order)
 *                         with need_logits
 *   counts[0]             N = sum of n;  counts[1] = number of logits indices.
 * All arrays are int32 device memory owned by the caller: positions and
 * slot_mapping hold max_tokens entries (tokens at or past max_tokens are not
 * written: check counts[0] <= max_tokens), logits_indices holds B entries.
 * block_tables is [B, bt_stride] with bt_cols valid columns per row.  Two kernels
 * on `stream`; no host synchronisation and no allocation, so the call can be
 * captured in a HIP graph and replayed with new inputs.  Arguments are checked
 * on the host; a failed check enqueues nothing. */
rpkv_status rpkv_build_metadata(int32_t batch, const int32_t *num_computed, const int32_t *n,
                                const uint8_t *need_logits, const int32_t *block_tables,
                                int64_t bt_stride, int32_t bt_cols, int32_t page_size,
                                int64_t max_tokens, int32_t *query_start_loc, int32_t *seq_lens,
                                int32_t *positions, int32_t *slot_mapping,
                                int32_t *logits_indices, int32_t *counts, void *stream);

/* ------------------------------------------------------- instrumentation */

/* Enable (1) or disable (0) per-launch HIP-event timing on this plan, with room
 * for max_launches launches before rpkv_timing_collect must be called. */
rpkv_status rpkv_timing_enable(rpkv_plan *plan, int32_t enable, int32_t max_launches);

/* Wait for the recorded events, add their durations into *out and reset the
 * record.  Blocks the host until the recorded launches finish. */
rpkv_status rpkv_timing_collect(rpkv_plan *plan, rpkv_kernel_times *out);

#ifdef __cplusplus
}
#endif

#endif /* RPKV_H */
