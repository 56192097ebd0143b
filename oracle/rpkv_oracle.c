/*
 * rpkv oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of what one step of ragged, paged,
 * prefix-cached causal attention computes.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the GPU library never does, and
 * the two share no code, headers or tables.
 *
 * What it follows (page title, then section):
 *  - mini-sglang "The attention backend and a reference implementation",
 *    "The interface": forward() writes this step's K/V into the pool first and
 *    only then reads the pool back (store before attend).
 *  - same page, "Variable-length, paged attention with prefixes": request i owns
 *    query rows [cu_q[i], cu_q[i+1]); its KV is the first cache_seqlens[i]
 *    locations named by its page-table row; the n queries are the last n
 *    positions, so query r sits at position L-n+r and sees keys 0..L-n+r
 *    (bottom-right alignment); scaled_dot_product_attention with enable_gqa
 *    shares each KV head among G = Hq/Hkv consecutive query heads.
 *  - "Variable-length batching and one mixed forward pass", "Layout and
 *    metadata" and "Implementation": positions, seq_lens, query_start_loc and
 *    logits_indices of a packed batch; slots come from the block table.
 *  - SGLang source walkthrough "Attention backends", 3.3 "Cascade Inference":
 *    a shared prefix and the unique tails are attended separately and merged by
 *    their log-sum-exp.  The page text lost the displayed formula; the merge here
 *    is the identity softmax over a disjoint union of key sets obeys.
 *
 * Readings of the pages where they are silent (each is listed in the design
 * notes): page-table entries are page ids and position x of request i lives in
 * slot row[x/P]*P + x%P (reduces to the page_size=1 example exactly); KV head of
 * query head h is h/G; softmax uses the natural exponential and the scale is an
 * explicit argument.
 *
 * All arithmetic is double precision on exactly up-cast inputs (bf16 arrives as
 * its 16-bit pattern, fp32 as float).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1 };

typedef struct {
  int32_t dtype;            /* ORACLE_BF16 or ORACLE_F32 */
  int32_t num_q_heads;      /* Hq */
  int32_t num_kv_heads;     /* Hkv, divides Hq */
  int32_t head_dim;         /* D */
  int32_t page_size;        /* P */
  int32_t batch;            /* bs */
  const int32_t *cu_q;      /* [bs+1] */
  const int32_t *seqlens;   /* [bs]  L_i, KV length including this step */
  const int32_t *page_table;/* [bs, stride] page ids */
  int64_t pt_stride;        /* elements between rows */
  const void *q;            /* [T, Hq, D] */
  const void *kpool;        /* [slots, Hkv, D] (after the store) */
  const void *vpool;
  double scale;
  int64_t key_lo;           /* only keys j in [key_lo, key_hi) are attended;  */
  int64_t key_hi;           /* the full definition uses [0, huge)             */
} oracle_problem;

static double up(const void *base, int64_t idx, int dtype) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float *)base)[idx];
}

/* Pool slot of logical position pos of request req: the page id in the row's
 * (pos / P)-th entry, times P, plus the offset pos % P. */
int64_t rpkv_oracle_slot(const int32_t *page_table, int64_t pt_stride, int32_t req, int64_t pos,
                         int32_t page_size) {
  int64_t page = page_table[(int64_t)req * pt_stride + pos / page_size];
  return page * page_size + pos % page_size;
}

/* Store: for each new token t in order, its K row and V row are copied bit for
 * bit into pool slot slot_mapping[t].  A negative slot is skipped. */
void rpkv_oracle_store_kv(void *kpool, void *vpool, const void *k, const void *v,
                          const int32_t *slot_mapping, int64_t T, int64_t row_bytes) {
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    memcpy((char *)kpool + s * row_bytes, (const char *)k + t * row_bytes, (size_t)row_bytes);
    memcpy((char *)vpool + s * row_bytes, (const char *)v + t * row_bytes, (size_t)row_bytes);
  }
}

/* last position of each request in the packed q (-1 for a request with no
 * queries this step) */
void rpkv_oracle_last_indices(const int32_t *cu_q, int32_t bs, int32_t *out) {
  for (int32_t i = 0; i < bs; ++i) out[i] = (cu_q[i + 1] > cu_q[i]) ? cu_q[i + 1] - 1 : -1;
}

/* Packed-batch metadata from per-request (num_computed, n, need_logits), as the
 * mixed-forward page builds it: positions num_computed..num_computed+n-1,
 * query_start_loc as the running sum of n, seq_len = num_computed + n, and the
 * last packed index of each request that needs logits.  Slots come from each
 * request's block table.  Returns the number of logits indices written. */
int32_t rpkv_oracle_build_batch(int32_t bs, const int32_t *num_computed, const int32_t *n,
                                const uint8_t *need_logits, const int32_t *block_tables,
                                int64_t bt_stride, int32_t block_size, int32_t *qsl,
                                int32_t *seq_lens, int32_t *positions, int32_t *slots,
                                int32_t *logits_idx) {
  int32_t t = 0, m = 0;
  qsl[0] = 0;
  for (int32_t i = 0; i < bs; ++i) {
    for (int32_t r = 0; r < n[i]; ++r) {
      int32_t pos = num_computed[i] + r;
      positions[t] = pos;
      if (block_tables)
        slots[t] = (int32_t)rpkv_oracle_slot(block_tables, bt_stride, i, pos, block_size);
      ++t;
    }
    qsl[i + 1] = t;
    seq_lens[i] = num_computed[i] + n[i];
    if (need_logits[i]) logits_idx[m++] = t - 1;
  }
  return m;
}

/* One (token, head) output: the definition written out.
 *   x_j = scale * <q[t,h,:], K[slot(i,j), h/G, :]>   for visible j
 *   out = sum_j exp(x_j - m) V[slot(i,j), h/G, :] / sum_j exp(x_j - m)
 *   lse = m + ln sum_j exp(x_j - m)
 * Visible keys: j <= L-n+r (bottom-right causal), intersected with
 * [key_lo, key_hi).  No visible key: out = 0 and lse = -inf. */
static void attend_one(const oracle_problem *pb, int32_t req, int32_t t, int32_t h, double *x,
                       double *out, double *lse) {
  const int32_t D = pb->head_dim, Hq = pb->num_q_heads, Hkv = pb->num_kv_heads;
  const int32_t G = Hq / Hkv, kvh = h / G;
  const int32_t n = pb->cu_q[req + 1] - pb->cu_q[req];
  const int64_t L = pb->seqlens[req];
  const int64_t r = t - pb->cu_q[req];
  const int64_t a = L - n + r; /* absolute position of this query */
  int64_t lo = pb->key_lo > 0 ? pb->key_lo : 0;
  int64_t hi = a + 1 < pb->key_hi ? a + 1 : pb->key_hi;
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (hi <= lo) {
    *lse = -INFINITY;
    return;
  }
  const int64_t qbase = ((int64_t)t * Hq + h) * D;
  double m = -INFINITY;
  for (int64_t j = lo; j < hi; ++j) {
    int64_t s = rpkv_oracle_slot(pb->page_table, pb->pt_stride, req, j, pb->page_size);
    int64_t kbase = (s * Hkv + kvh) * D;
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d) dot += up(pb->q, qbase + d, pb->dtype) * up(pb->kpool, kbase + d, pb->dtype);
    x[j - lo] = pb->scale * dot;
    if (x[j - lo] > m) m = x[j - lo];
  }
  double Z = 0.0;
  for (int64_t j = lo; j < hi; ++j) {
    int64_t s = rpkv_oracle_slot(pb->page_table, pb->pt_stride, req, j, pb->page_size);
    int64_t vbase = (s * Hkv + kvh) * D;
    double w = exp(x[j - lo] - m);
    Z += w;
    for (int32_t d = 0; d < D; ++d) out[d] += w * up(pb->vpool, vbase + d, pb->dtype);
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= Z;
  *lse = m + log(Z);
}

typedef struct {
  const oracle_problem *pb;
  const uint8_t *row_sel; /* [T] or NULL: which tokens to compute */
  const int32_t *tok_req; /* [T] request of each token */
  double *out, *lse;
  int64_t T;
  int32_t tid, nthreads;
  int64_t max_len;
} worker_arg;

static void *worker(void *p) {
  worker_arg *w = (worker_arg *)p;
  const oracle_problem *pb = w->pb;
  double *x = (double *)malloc(sizeof(double) * (size_t)(w->max_len > 0 ? w->max_len : 1));
  const int32_t Hq = pb->num_q_heads, D = pb->head_dim;
  for (int64_t t = w->tid; t < w->T; t += w->nthreads) {
    if (w->row_sel && !w->row_sel[t]) continue;
    for (int32_t h = 0; h < Hq; ++h)
      attend_one(pb, w->tok_req[t], (int32_t)t, h, x, w->out + ((int64_t)t * Hq + h) * D,
                 w->lse + (int64_t)t * Hq + h);
  }
  free(x);
  return NULL;
}

/* Attention of every (selected) token and head.  out: [T, Hq, D] doubles, lse:
 * [T, Hq] doubles.  Rows not selected are left untouched.  Returns 0, or -1 on
 * an input the definition does not cover (n > L, non-monotone cu_q, Hq % Hkv). */
int32_t rpkv_oracle_attend(const oracle_problem *pb, const uint8_t *row_sel, double *out,
                           double *lse, int32_t nthreads) {
  if (pb->num_kv_heads <= 0 || pb->num_q_heads % pb->num_kv_heads) return -1;
  if (pb->cu_q[0] != 0) return -1;
  int64_t T = pb->cu_q[pb->batch], max_len = 1;
  for (int32_t i = 0; i < pb->batch; ++i) {
    int32_t n = pb->cu_q[i + 1] - pb->cu_q[i];
    if (n < 0 || n > pb->seqlens[i]) return -1;
    if (pb->seqlens[i] > max_len) max_len = pb->seqlens[i];
  }
  int32_t *tok_req = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  for (int32_t i = 0; i < pb->batch; ++i)
    for (int32_t t = pb->cu_q[i]; t < pb->cu_q[i + 1]; ++t) tok_req[t] = i;
  if (nthreads < 1) nthreads = 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  worker_arg *args = (worker_arg *)malloc(sizeof(worker_arg) * (size_t)nthreads);
  for (int32_t k = 0; k < nthreads; ++k) {
    args[k] = (worker_arg){pb, row_sel, tok_req, out, lse, T, k, nthreads, max_len};
    if (nthreads == 1) worker(&args[k]);
    else pthread_create(&th[k], NULL, worker, &args[k]);
  }
  if (nthreads > 1)
    for (int32_t k = 0; k < nthreads; ++k) pthread_join(th[k], NULL);
  free(args);
  free(th);
  free(tok_req);
  return 0;
}

/* Merge of partial results over disjoint key sets (cascade 3.3, and split-KV
 * decoding).  For each row with partials (o_s, lse_s):
 *   lse = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - lse) o_s.
 * Evaluated with the largest lse_s factored out; a partial with lse_s = -inf has
 * weight 0; a row with no finite partial gets out = 0, lse = -inf.
 * o_parts: [nparts, rows, D], lse_parts: [nparts, rows]. */
void rpkv_oracle_lse_merge(int32_t nparts, int64_t rows, int32_t D, const double *o_parts,
                           const double *lse_parts, double *out, double *lse_out) {
  for (int64_t r = 0; r < rows; ++r) {
    double M = -INFINITY;
    for (int32_t s = 0; s < nparts; ++s)
      if (lse_parts[s * rows + r] > M) M = lse_parts[s * rows + r];
    for (int32_t d = 0; d < D; ++d) out[r * D + d] = 0.0;
    if (M == -INFINITY) {
      lse_out[r] = -INFINITY;
      continue;
    }
    double W = 0.0;
    for (int32_t s = 0; s < nparts; ++s) {
      double l = lse_parts[s * rows + r];
      if (l == -INFINITY) continue;
      double w = exp(l - M);
      W += w;
      for (int32_t d = 0; d < D; ++d) out[r * D + d] += w * o_parts[(s * rows + r) * D + d];
    }
    for (int32_t d = 0; d < D; ++d) out[r * D + d] /= W;
    lse_out[r] = M + log(W);
  }
}
