// Host planner: turns one batch's metadata into the work partition the kernels
// consume.  Runs once per batch and serves every layer (mini-sglang "The
// attention backend and a reference implementation", "The interface"; vLLM
// "Attention backends", Step 5: one metadata object for all layers of a group).
//
// What it decides:
//  * classification: a request whose n * G query rows fit one 16-column MFMA
//    tile is decode-type and runs on the split-KV kernel; the others are
//    prefill-type and run on 128-row MFMA tiles (SGLang walkthrough, section 6:
//    a mixed batch is split by token between decode and prefill work; "Variable-
//    length batching and one mixed forward pass", exercise 2: decode work uses
//    split-KV kernels);
//  * prefill tiles: 128 / G tokens x G heads of one KV head per tile, key range
//    cut at the tile's last causal position (bottom-right mask);
//  * split-KV chunks: one chunk length for the whole batch, chosen ahead of time
//    so the decode launch has about `split_target` items (vLLM's FlashAttention
//    metadata carries ahead-of-time scheduler data and a split count);
//  * cascade: a tree of shared-prefix levels, from nested hints or found in the
//    host page table (radix tree of the decode requests' cached page ids); each
//    level's eligible members are stacked in tiles against the keys the level
//    adds, each member keeps its own tail chunks, and the partials along a
//    member's path are merged by log-sum-exp (SGLang walkthrough 3.3; the
//    multi-level form takes one level per depth of the radix tree);
//  * partial-result layout and the merge list;
//  * launch order: prefill tiles that read the same K/V go to the same XCD
//    (blocks are dealt round-robin to the 8 XCDs, each with its own L2), and
//    each XCD's queue runs longest work first.
#include <algorithm>
#include <climits>
#include <chrono>
#include <cstring>
#include <numeric>
#include <string>
#include <tuple>

#include "rpkv_internal.h"

namespace rpkv {

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

rpkv_status check_shape(const rpkv_shape *s, Shape *o, std::string *msg) {
  if (!s) {
    *msg = "shape is NULL";
    return RPKV_ERR_INVALID_ARG;
  }
  if (s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->num_q_heads % s->num_kv_heads) {
    *msg = "num_q_heads and num_kv_heads must be positive and Hq % Hkv == 0";
    return RPKV_ERR_INVALID_ARG;
  }
  if (s->num_q_heads / s->num_kv_heads > kPrefillRows) {
    *msg = "Hq / Hkv above 128 is not supported";
    return RPKV_ERR_UNSUPPORTED;
  }
  if (s->dtype != RPKV_BF16 && s->dtype != RPKV_F32) {
    *msg = "dtype must be RPKV_BF16 or RPKV_F32";
    return RPKV_ERR_INVALID_ARG;
  }
  if (s->head_dim <= 0) {
    *msg = "head_dim must be positive";
    return RPKV_ERR_INVALID_ARG;
  }
  if (s->dtype == RPKV_BF16 && s->head_dim != 128) {
    *msg = "bf16 kernels are built for head_dim 128";
    return RPKV_ERR_UNSUPPORTED;
  }
  if (s->dtype == RPKV_F32 && s->num_q_heads / s->num_kv_heads > kF32Rows) {
    *msg = "fp32 kernels serve Hq / Hkv <= 16 (one 16-row tile per token)";
    return RPKV_ERR_UNSUPPORTED;
  }
  if (s->dtype == RPKV_F32 && s->head_dim != 64 && s->head_dim != 128) {
    *msg = "fp32 kernels are built for head_dim 64 and 128";
    return RPKV_ERR_UNSUPPORTED;
  }
  if (s->page_size < 1 || s->page_size > 1024 || (s->page_size & (s->page_size - 1))) {
    *msg = "page_size must be a power of two in [1, 1024]";
    return RPKV_ERR_UNSUPPORTED;
  }
  if (s->max_batch <= 0 || s->num_pages <= 0 || s->max_tokens <= 0 ||
      s->max_pages_per_req <= 0) {
    *msg = "max_batch, num_pages, max_tokens and max_pages_per_req must be positive";
    return RPKV_ERR_INVALID_ARG;
  }
  if (s->num_pages * (int64_t)s->page_size > INT32_MAX || s->max_tokens > INT32_MAX ||
      (int64_t)s->max_pages_per_req * s->page_size > INT32_MAX) {
    *msg = "slots, tokens and sequence lengths must fit int32";
    return RPKV_ERR_INVALID_ARG;
  }
  if (s->decode_max_rows < 0 || s->decode_max_rows > kDecodeRows || s->split_target < 0 ||
      s->split_min_keys < 0 || s->prefix_detect_keys < 0 || s->tiles_per_block < 0 ||
      s->tiles_per_block > 2) {
    *msg = "tuning fields out of range (decode_max_rows <= 16, tiles_per_block <= 2, others >= 0)";
    return RPKV_ERR_INVALID_ARG;
  }
  o->Hq = s->num_q_heads;
  o->Hkv = s->num_kv_heads;
  o->D = s->head_dim;
  o->P = s->page_size;
  o->log2P = 0;
  while ((1 << o->log2P) < s->page_size) ++o->log2P;
  o->dtype = s->dtype;
  o->max_batch = s->max_batch;
  o->max_pages_per_req = s->max_pages_per_req;
  o->num_pages = s->num_pages;
  o->max_tokens = s->max_tokens;
  o->decode_max_rows = s->decode_max_rows ? s->decode_max_rows : kDecodeRows;
  o->split_target = s->split_target ? s->split_target : 3072;
  o->split_min_keys = (int32_t)round_up(s->split_min_keys ? s->split_min_keys : 64, kDecodeKeys);
  o->prefix_detect_keys = s->prefix_detect_keys;
  o->tiles_per_block = s->tiles_per_block;
  o->check_slots = s->check_slots;
  return RPKV_OK;
}

void graph_decode_chunks(int64_t max_batch, int32_t Hkv, int32_t max_seq, int32_t *chunk,
                         int32_t *maxc) {
  const int64_t waves_per_chunk = std::max<int64_t>(1, max_batch * Hkv);
  const int64_t want = std::min<int64_t>(32, std::max<int64_t>(2, cdiv(8192, waves_per_chunk)));
  *chunk = (int32_t)std::max<int64_t>(256, round_up(cdiv(max_seq, want), 64));
  *maxc = (int32_t)cdiv(max_seq, *chunk);
}

// Slots are sorted together with their token index (packed in one 64-bit key),
// so equal neighbours name a duplicate and its first two tokens.
int64_t find_bad_slot(const int32_t *slots, int64_t n, int64_t num_slots,
                      std::vector<int64_t> *scratch, std::string *msg) {
  if (n > INT32_MAX) {
    *msg = "slot_mapping longer than 2^31 - 1 tokens";
    return 0;
  }
  std::vector<int64_t> &key = *scratch;
  key.clear();
  for (int64_t t = 0; t < n; ++t) {
    const int32_t s = slots[t];
    if (s < 0) continue;  // padding token
    if (s >= num_slots) {
      *msg = "slot_mapping[" + std::to_string(t) + "] = " + std::to_string(s) +
             " is outside the pool of " + std::to_string(num_slots) + " slots";
      return t;
    }
    key.push_back(((int64_t)s << 32) | t);
  }
  std::sort(key.begin(), key.end());
  int64_t bad = -1, first = -1;
  for (size_t k = 1; k < key.size(); ++k)
    if ((key[k] >> 32) == (key[k - 1] >> 32)) {
      const int64_t a = key[k - 1] & 0xFFFFFFFF, b = key[k] & 0xFFFFFFFF;
      if (bad < 0 || b < bad) {
        bad = b;
        first = a;
      }
    }
  if (bad >= 0)
    *msg = "slot_mapping[" + std::to_string(bad) + "] repeats the slot of token " +
           std::to_string(first) + " (" + std::to_string(slots[bad]) + ")";
  return bad;
}

// Bounds on the work partition of any batch within the shape's capacities
// (B requests, Tm tokens, rows of at most Lmax keys), following the rules below:
//  * prefill-type tiles: sum over requests of ceil(n / tpt) per KV head, at most
//    (ceil(Tm / tpt) + B) * Hkv; key splits make at most twice that plus
//    kPrefillSlots pieces (a tile becomes at most s / fair + 1 pieces, s the
//    steps of the longer of it and its sibling, at most 3 more than its own,
//    fair >= 8 and >= total steps / 512);
//  * cascade: a level holds decode-type tokens (n * G <= decode_max_rows), each
//    in at most kMaxCascadeDepth levels, and there are fewer than B levels; the
//    level tiles are at most kPrefillSlots + (tokens / tpt + levels) * Hkv (the
//    level chunk is at least the levels' work / 512);
//  * the XCD order pads to at most 2 * items + 16 single items, or 2 * units + 8
//    workgroups of two siblings (units <= items), i.e. 4 * items + 16;
//  * split-KV chunks: at most decode keys / chunk + one short chunk per
//    (request, KV head), with chunk >= decode keys / split_target and >=
//    split_min_keys;
//  * per token one partial base and at most one merge record of 3 entries.
MetaCounts meta_caps(const Shape &s) {
  const int64_t G = s.G(), B = s.max_batch, Tm = s.max_tokens, Hkv = s.Hkv;
  const int64_t tpt = std::max<int64_t>(1, (s.dtype == RPKV_F32 ? kF32Rows : kPrefillRows) / G);
  const int64_t Lmax = (int64_t)s.max_pages_per_req * s.P;
  const int64_t pieces = 2 * (cdiv(Tm, tpt) + B) * Hkv + kPrefillSlots;
  const int64_t dtok = std::min<int64_t>(Tm, B * (s.decode_max_rows / G));
  const int64_t tok = dtok * kMaxCascadeDepth;
  const int64_t lev_tiles = tok > 0 ? kPrefillSlots + (cdiv(tok, tpt) + B) * Hkv : 0;
  MetaCounts c{};
  c.pre = 4 * (pieces + lev_tiles) + 2 * kNumXcd;
  // B, Lmax and Hkv are each below 2^31: B * Lmax fits, the product with Hkv may not
  const int64_t keys = B * Lmax;
  const int64_t chunks = keys > INT64_MAX / Hkv ? INT64_MAX : cdiv(keys * Hkv, s.split_min_keys);
  c.dec = dtok > 0 ? std::min<int64_t>(s.split_target, chunks) + B * Hkv : 0;
  c.pbase = Tm;
  c.merge = 3 * Tm;
  c.tok = tok;
  c.indptr = B + 1;
  return c;
}

MetaCounts meta_counts(const HostPlan &p, int32_t max_batch) {
  MetaCounts c{};
  c.pre = (int64_t)p.prefill.size();
  c.dec = (int64_t)p.decode.size();
  c.pbase = (int64_t)p.tok_pbase.size();
  c.merge = (int64_t)p.merge.size();
  c.tok = (int64_t)p.toklist.size();
  c.indptr = (int64_t)max_batch + 1;  // room for a CSR table's row offsets
  return c;
}

// The device copy: items, split-KV items, token partial bases, merge records,
// cascade token lists, CSR row offsets; each array 256-byte aligned.
MetaLayout meta_layout(const MetaCounts &c) {
  auto a256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  MetaLayout l{};
  size_t off = 0;
  l.off_pre = off;
  off = a256(off + (size_t)c.pre * sizeof(Item));
  l.off_dec = off;
  off = a256(off + (size_t)c.dec * sizeof(Item));
  l.off_pbase = off;
  off = a256(off + (size_t)c.pbase * sizeof(int32_t));
  l.off_merge = off;
  off = a256(off + (size_t)c.merge * sizeof(int32_t));
  l.off_tok = off;
  off = a256(off + (size_t)c.tok * sizeof(int32_t));
  l.off_indptr = off;
  off = a256(off + (size_t)c.indptr * sizeof(int32_t));
  l.bytes = std::max<size_t>(off, 256);
  return l;
}

namespace {

int64_t item_work(const Item &it) {
  // key tiles touched; every tile costs the same MFMA work for a full tile
  return it.ntok ? cdiv(std::max(it.kend - it.kbeg, 1), kPrefillKeys) : 0;
}

// Deal prefill items to per-XCD queues: items sharing K/V (same group key)
// stay on one XCD, groups larger than a fair share are cut into contiguous
// pieces, pieces are placed longest-first on the least loaded queue, each queue
// runs longest-first, and the queues are interleaved so block b runs on XCD b%8.
// The result is the launch order as indices into the items, -1 for padding.
void xcd_order(const std::vector<int64_t> &work, const std::vector<int64_t> &gkey, int per_block,
               std::vector<int32_t> *outp) {
  std::vector<int32_t> &out = *outp;
  out.clear();
  if (work.empty()) return;
  const size_t n = work.size();
  // items sharing K/V together, in ascending key order (the planner emits them
  // that way, so this is usually the identity); ties keep the input order
  std::vector<size_t> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  if (!std::is_sorted(gkey.begin(), gkey.end()))
    std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return gkey[a] < gkey[b]; });
  // dense rank of each item's key (ascending keys -> ascending ranks)
  std::vector<uint32_t> grank(n);
  for (size_t k = 0, r = 0; k < n; ++k) {
    if (k > 0 && gkey[idx[k]] != gkey[idx[k - 1]]) ++r;
    grank[idx[k]] = (uint32_t)r;
  }
  int64_t total = 0;
  for (int64_t w : work) total += w;
  const int64_t share = std::max<int64_t>(1, cdiv(total, kNumXcd));
  struct Piece {
    std::vector<size_t> members;
    int64_t work = 0;
  };
  std::vector<Piece> pieces;
  size_t i = 0;
  while (i < n) {
    size_t j = i;
    int64_t gw = 0;
    while (j < n && gkey[idx[j]] == gkey[idx[i]]) gw += work[idx[j++]];
    const int64_t npieces = std::max<int64_t>(1, cdiv(gw, share));
    const int64_t per = cdiv(gw, npieces);
    Piece cur;
    for (size_t k = i; k < j; ++k) {
      cur.members.push_back(idx[k]);
      cur.work += work[idx[k]];
      if (cur.work >= per) {
        pieces.push_back(std::move(cur));
        cur = Piece();
      }
    }
    if (!cur.members.empty()) pieces.push_back(std::move(cur));
    i = j;
  }
  std::vector<size_t> porder(pieces.size());
  std::iota(porder.begin(), porder.end(), 0);
  std::sort(porder.begin(), porder.end(), [&](size_t a, size_t b) {
    return pieces[a].work != pieces[b].work ? pieces[a].work > pieces[b].work : a < b;
  });
  std::vector<std::vector<size_t>> q(kNumXcd);
  std::vector<int64_t> load(kNumXcd, 0);
  for (size_t pi : porder) {
    Piece &p = pieces[pi];
    int best = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[best] += p.work;
    q[best].insert(q[best].end(), p.members.begin(), p.members.end());
  }
  // Every queue is padded to the longest one's length; when the queues' item
  // counts are very unequal (many short items against a few long ones) the
  // shortest items of the fullest queues move to the emptiest, so the padded
  // list holds at most 2 * n + 8 * per_block items (the plan's metadata buffer
  // is sized for that bound).
  {
    const size_t cap = (size_t)round_up(cdiv((int64_t)(2 * n), kNumXcd), per_block);
    size_t longest = 0;
    for (auto &qq : q) longest = std::max(longest, qq.size());
    if (longest > cap) {
      for (int x = 0; x < kNumXcd; ++x) {
        // the queue's items, shortest last
        std::stable_sort(q[x].begin(), q[x].end(),
                         [&](size_t a, size_t b) { return work[a] > work[b]; });
      }
      for (int x = 0; x < kNumXcd; ++x)
        while (q[x].size() > cap) {
          int y = 0;
          for (int z = 1; z < kNumXcd; ++z)
            if (q[z].size() < q[y].size()) y = z;
          q[y].push_back(q[x].back());
          q[x].pop_back();
        }
    }
  }
  // Within a queue: longest first by coarse work bucket (eighths of the queue's
  // longest item), and inside a bucket tiles sharing K/V together, so nearly
  // equal tiles of one group run side by side and their K/V stays in the XCD's
  // L2, while very unequal tiles still start longest first.  (The members of a
  // piece were appended in group order; the sort key decides everything else.)
  // The order is packed into one 64-bit key per item (bucket descending, key rank
  // ascending, work descending) with the item index as the final tie-break.
  size_t qlen = 0;
  std::vector<std::pair<uint64_t, uint32_t>> keyed;
  for (auto &qq : q) {
    int64_t mx = 1;
    for (size_t k : qq) mx = std::max(mx, work[k]);
    keyed.clear();
    keyed.reserve(qq.size());
    for (size_t k : qq) {
      const uint64_t b = (uint64_t)(work[k] * 8 / (mx + 1));  // 0..7
      const uint64_t w = (uint64_t)std::min<int64_t>(work[k], 0xFFFFFFFF);
      keyed.emplace_back(((7 - b) << 60) | ((uint64_t)std::min<uint32_t>(grank[k], 0x0FFFFFFF) << 32) |
                             (0xFFFFFFFF - w),
                         (uint32_t)k);
    }
    std::sort(keyed.begin(), keyed.end());
    for (size_t k = 0; k < qq.size(); ++k) qq[k] = keyed[k].second;
    qlen = std::max(qlen, qq.size());
  }
  // workgroup b runs on XCD b % 8 and takes per_block consecutive items:
  // items k..k+per_block-1 of queue x go to workgroup (k / per_block) * 8 + x
  const size_t per = (size_t)per_block;
  qlen = (qlen + per - 1) / per * per;
  out.assign(qlen * kNumXcd, -1);
  for (int x = 0; x < kNumXcd; ++x)
    for (size_t k = 0; k < q[x].size(); ++k)
      out[((k / per) * kNumXcd + x) * per + k % per] = (int32_t)q[x][k];
}

// A candidate level: positions [lb, lb + cnt) of a request order share `prefix`
// keys.
struct Span {
  int32_t lb, cnt, prefix;
};

// Shared-prefix detection (SGLang walkthrough "Attention backends", 3.2: the
// radix cache fills the page table, so requests that reuse a cached prefix carry
// its page ids; 3.3: the multi-level cascade takes one level per depth of the
// radix tree).  Request j offers its first offered(j) page ids -- the pages whose
// keys were all cached before this step.  The radix tree of the offered
// sequences is grown top-down: a group of requests known to agree on `depth` ids
// extends `depth` while all of them agree on the next id (that depth, in keys,
// is the group's shared prefix and the group a candidate level if it is not the
// root), then splits by the next id, requests whose sequence ends there leaving
// the group; each part of two or more is grown the same way.  The work is the
// number of (member, shared page) pairs plus a sort at each branch point.
// Candidates are spans of `order`, which ends up grouped by tree position.
template <class Offered>
void detect_shared_prefixes(int32_t P, int32_t batch, int32_t cols, const int32_t *pt,
                            Offered offered, std::vector<int32_t> *order,
                            std::vector<Span> *spans) {
  std::vector<int32_t> len(batch, 0);
  order->clear();
  for (int32_t j = 0; j < batch; ++j) {
    len[j] = std::min(offered(j), cols);
    if (len[j] > 0) order->push_back(j);
  }
  std::vector<int32_t> &ord = *order;
  auto id_at = [&](int32_t j, int32_t d) {  // -1 once the sequence has ended
    return d < len[j] ? pt[(int64_t)j * cols + d] : -1;
  };
  struct Group {
    int32_t lb, ub, depth;
  };
  std::vector<Group> work;
  if (ord.size() >= 2) work.push_back(Group{0, (int32_t)ord.size(), 0});
  while (!work.empty()) {
    Group g = work.back();
    work.pop_back();
    for (;;) {
      const int32_t id = id_at(ord[g.lb], g.depth);
      if (id < 0) break;
      int32_t k = g.lb + 1;
      while (k < g.ub && id_at(ord[k], g.depth) == id) ++k;
      if (k < g.ub) break;
      ++g.depth;
    }
    if (g.depth > 0) spans->push_back(Span{g.lb, g.ub - g.lb, g.depth * P});
    std::sort(ord.begin() + g.lb, ord.begin() + g.ub, [&](int32_t a, int32_t b) {
      const int32_t ia = id_at(a, g.depth), ib = id_at(b, g.depth);
      return ia != ib ? ia < ib : a < b;
    });
    // parts in reverse so the stack grows them in order (parents before children)
    for (int32_t e = g.ub; e > g.lb;) {
      int32_t b = e - 1;
      const int32_t id = id_at(ord[b], g.depth);
      while (b > g.lb && id_at(ord[b - 1], g.depth) == id) --b;
      if (id >= 0 && e - b >= 2) work.push_back(Group{b, e, g.depth + 1});
      e = b;
    }
  }
}

// Turns candidate levels into the level tree.  Candidates must nest (a range
// inside another has a longer prefix; ranges may not overlap otherwise).  A
// candidate becomes a level when at least two of its requests are eligible for
// its prefix, it adds at least min_keys keys to the nearest level above it, and
// it lies at most kMaxCascadeDepth levels deep; otherwise its nested candidates
// attach to that level (its keys then fall to the next level down or to the
// members' own tails: the same result, read less often shared).  Levels come out parents
// first, members ascending.
template <class Eligible>
rpkv_status nest_levels(std::vector<Span> spans, const std::vector<int32_t> &order,
                        Eligible eligible, int32_t min_keys, std::vector<CascNode> *tree,
                        std::string *msg) {
  std::sort(spans.begin(), spans.end(), [](const Span &a, const Span &b) {
    if (a.lb != b.lb) return a.lb < b.lb;
    if (a.cnt != b.cnt) return a.cnt > b.cnt;
    return a.prefix < b.prefix;
  });
  struct Open {
    int32_t end, prefix, level;  // level: nearest level at or above, or -1
  };
  std::vector<Open> st;
  std::vector<int32_t> depth;  // nesting depth of each level (1 at the top)
  tree->clear();
  for (const Span &sp : spans) {
    while (!st.empty() && st.back().end <= sp.lb) st.pop_back();
    const int32_t end = sp.lb + sp.cnt;
    int32_t above = -1;
    if (!st.empty()) {
      if (end > st.back().end) {
        *msg = "cascade groups overlap without nesting (at request order position " +
               std::to_string(sp.lb) + ")";
        return RPKV_ERR_INVALID_ARG;
      }
      if (sp.prefix <= st.back().prefix) {
        *msg = "a nested cascade group needs a longer prefix than the group enclosing it";
        return RPKV_ERR_INVALID_ARG;
      }
      above = st.back().level;
    }
    const int32_t base = above >= 0 ? (*tree)[above].prefix : 0;
    std::vector<int32_t> members;
    for (int32_t k = sp.lb; k < end; ++k)
      if (eligible(order[k], sp.prefix)) members.push_back(order[k]);
    int32_t level = above;
    const int32_t d = above >= 0 ? depth[above] + 1 : 1;
    if (members.size() >= 2 && sp.prefix - base >= min_keys && d <= kMaxCascadeDepth) {
      std::sort(members.begin(), members.end());
      tree->push_back(CascNode{above, sp.prefix, std::move(members)});
      depth.push_back(d);
      level = (int32_t)tree->size() - 1;
    }
    st.push_back(Open{end, sp.prefix, level});
  }
  return RPKV_OK;
}

}  // namespace

rpkv_status plan_batch_host(const Shape &s, int32_t batch, const int32_t *cu, const int32_t *L,
                            int32_t cols, const int32_t *pt_host, const rpkv_prefix_group *groups,
                            int32_t ngroups, HostPlan *out, std::string *msg) {
  auto t_start = std::chrono::steady_clock::now();
  HostPlan &p = *out;  // the caller's scratch plan; on an error its contents are unspecified
  p.reset();
  // ------------------------------------------------------------ validation
  if (batch < 0) {
    *msg = "batch must be >= 0";
    return RPKV_ERR_INVALID_ARG;
  }
  if (batch > s.max_batch) {
    *msg = "batch exceeds the plan's max_batch";
    return RPKV_ERR_CAPACITY;
  }
  if (!cu) {
    *msg = "cu_seqlens_q_host is NULL";
    return RPKV_ERR_INVALID_ARG;
  }
  if (batch > 0 && !L) {
    *msg = "cache_seqlens_host is NULL";
    return RPKV_ERR_INVALID_ARG;
  }
  if (cu[0] != 0) {
    *msg = "cu_seqlens_q[0] must be 0";
    return RPKV_ERR_INVALID_ARG;
  }
  if (cols < 0 || ngroups < 0 || (ngroups > 0 && !groups)) {
    *msg = "page_table_cols and num_groups must be >= 0 (groups non-NULL when num_groups > 0)";
    return RPKV_ERR_INVALID_ARG;
  }
  if (cols > s.max_pages_per_req) {
    *msg = "page_table_cols exceeds the plan's max_pages_per_req";
    return RPKV_ERR_CAPACITY;
  }
  for (int32_t i = 0; i < batch; ++i) {
    const int64_t n = (int64_t)cu[i + 1] - cu[i];
    if (n < 0) {
      *msg = "cu_seqlens_q must be non-decreasing (request " + std::to_string(i) + ")";
      return RPKV_ERR_INVALID_ARG;
    }
    if (L[i] < 0 || n > L[i]) {
      *msg = "request " + std::to_string(i) + " has more queries than KV (n > L) or L < 0";
      return RPKV_ERR_INVALID_ARG;
    }
    if (cdiv(L[i], s.P) > cols) {
      *msg = "request " + std::to_string(i) + " needs more page-table columns than given";
      return RPKV_ERR_INVALID_ARG;
    }
  }
  const int64_t T64 = batch ? cu[batch] : 0;
  if (T64 > s.max_tokens) {
    *msg = "number of tokens exceeds the plan's max_tokens";
    return RPKV_ERR_CAPACITY;
  }
  if (pt_host) {
    for (int32_t i = 0; i < batch; ++i)
      for (int64_t c = 0; c < cdiv(L[i], s.P); ++c) {
        const int32_t id = pt_host[(int64_t)i * cols + c];
        if (id < 0 || id >= s.num_pages) {
          *msg = "page id out of [0, num_pages) in row " + std::to_string(i);
          return RPKV_ERR_INVALID_ARG;
        }
      }
  }
  for (int32_t g = 0; g < ngroups; ++g) {
    const rpkv_prefix_group &gr = groups[g];
    if (gr.first_req < 0 || gr.num_reqs < 0 || (int64_t)gr.first_req + gr.num_reqs > batch ||
        gr.prefix_len < 0 || gr.prefix_len % s.P) {
      *msg = "cascade group " + std::to_string(g) +
             " out of range or prefix_len not a multiple of page_size";
      return RPKV_ERR_INVALID_ARG;
    }
    if (!pt_host || gr.prefix_len == 0) continue;
    int32_t ref = -1;  // first member holding the whole prefix
    for (int32_t j = gr.first_req; j < gr.first_req + gr.num_reqs; ++j) {
      if (L[j] < gr.prefix_len) continue;
      if (ref < 0) {
        ref = j;
        continue;
      }
      for (int64_t c = 0; c < gr.prefix_len / s.P; ++c)
        if (pt_host[(int64_t)j * cols + c] != pt_host[(int64_t)ref * cols + c]) {
          *msg = "cascade group " + std::to_string(g) + ": request " + std::to_string(j) +
                 " does not share the prefix pages";
          return RPKV_ERR_INVALID_ARG;
        }
    }
  }

  // ------------------------------------------------------------ metadata
  const int32_t T = (int32_t)T64;
  const int32_t G = s.G();
  p.batch = batch;
  p.T = T;
  p.cu_q.assign(cu, cu + batch + 1);
  p.L.assign(L, L + batch);
  for (int32_t i = 0; i < batch; ++i) {
    p.max_q = std::max(p.max_q, cu[i + 1] - cu[i]);
    p.max_k = std::max(p.max_k, L[i]);
  }
  const bool f32 = s.dtype == RPKV_F32;
  const int32_t tile_rows = f32 ? kF32Rows : kPrefillRows;
  const int32_t tpt = std::max(1, tile_rows / G);  // tokens per prefill tile
  auto n_of = [&](int32_t i) { return cu[i + 1] - cu[i]; };
  auto is_decode = [&](int32_t i) {
    return n_of(i) > 0 && (int64_t)n_of(i) * G <= s.decode_max_rows;
  };

  // shared-prefix levels: from the hints, else detected from the page table
  auto eligible = [&](int32_t j, int32_t prefix) {
    return is_decode(j) && L[j] - n_of(j) >= prefix;
  };
  {
    std::vector<Span> spans;
    std::vector<int32_t> order;
    int32_t min_keys = 1;
    if (ngroups > 0) {
      order.resize(batch);
      std::iota(order.begin(), order.end(), 0);
      for (int32_t g = 0; g < ngroups; ++g)
        if (groups[g].num_reqs > 0 && groups[g].prefix_len > 0)
          spans.push_back(Span{groups[g].first_req, groups[g].num_reqs, groups[g].prefix_len});
    } else if (s.prefix_detect_keys > 0 && pt_host) {
      detect_shared_prefixes(s.P, batch, cols, pt_host, [&](int32_t j) {
        return is_decode(j) ? (L[j] - n_of(j)) / s.P : 0;
      }, &order, &spans);
      min_keys = s.prefix_detect_keys;
    }
    rpkv_status st = nest_levels(spans, order, eligible, min_keys, &p.tree, msg);
    if (st != RPKV_OK) return st;
  }
  const int32_t nlev = (int32_t)p.tree.size();
  std::vector<int32_t> &deepest = p.tmp.deepest;  // deepest level of each request
  deepest.assign(batch, -1);
  for (int32_t g = 0; g < nlev; ++g)
    for (int32_t j : p.tree[g].members) deepest[j] = g;
  auto own_from = [&](int32_t j) { return deepest[j] >= 0 ? p.tree[deepest[j]].prefix : 0; };
  for (int32_t g = 0; g < nlev; ++g) {
    int32_t d = 1;
    for (int32_t a = p.tree[g].parent; a >= 0; a = p.tree[a].parent) ++d;
    p.cascade_depth = std::max(p.cascade_depth, d);
  }

  std::vector<int32_t> &nsplit = p.tmp.nsplit;
  nsplit.assign(T, 1);
  std::vector<Item> &pre = p.tmp.pre, &dec = p.tmp.dec;
  std::vector<int64_t> &pre_key = p.tmp.pre_key;  // K/V-sharing group key per prefill item
  pre.clear();
  dec.clear();
  pre_key.clear();

  // prefill-type requests: tiles of tpt tokens x G heads of one KV head
  std::vector<Item> &tiles = p.tmp.tiles;
  std::vector<int64_t> &tile_key = p.tmp.tile_key;
  tiles.clear();
  tile_key.clear();
  {
    int64_t nt = 0;
    for (int32_t i = 0; i < batch; ++i)
      if (n_of(i) > 0 && !is_decode(i)) nt += cdiv(n_of(i), tpt) * s.Hkv;
    tiles.reserve(nt);
    tile_key.reserve(nt);
    pre.reserve(nt + nt / 2);
    pre_key.reserve(nt + nt / 2);
  }
  // the steps of the token-aligned tiles set the fair share of the key splits
  int64_t total_steps = 0;
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t n = n_of(i);
    if (n == 0 || is_decode(i)) continue;
    for (int32_t r0 = 0; r0 < n; r0 += tpt)
      total_steps += cdiv(L[i] - n + std::min(n, r0 + tpt), kPrefillKeys) * s.Hkv;
  }
  // A tile much longer than the fair share of steps per concurrent tile slot
  // would set the launch's critical path: cut its key range into pieces of whole
  // 64-key steps, merged afterwards like split-KV chunks.  (Not for fp32.)
  // Sibling tiles (consecutive row blocks of one request and KV head) are cut
  // at the same keys, from the longer one's length, so a workgroup running two
  // of them can share one K/V stream.
  const int64_t fair = std::max<int64_t>(8, cdiv(total_steps, kPrefillSlots));
  auto never_split = [&](int32_t i) { return cdiv(L[i], kPrefillKeys) <= fair + fair / 2; };
  // Tiles hold 128 / G whole tokens, except where G does not divide 128 and no
  // tile of the request is split: there the tiles cut the request's (token,
  // head) rows every 128 rows, so a token's heads may straddle two tiles (a
  // split tile's partials are counted per token, hence whole tokens there).
  // For G = 7 a 512-token chunk then takes 28 tiles of 128 rows instead of 29
  // of 18 tokens (the last holding 8).
  for (int32_t i = 0; i < batch; ++i) {
    const int32_t n = n_of(i);
    if (n == 0 || is_decode(i)) continue;
    const bool rowcut = !f32 && kPrefillRows % G != 0 && never_split(i);
    for (int32_t h = 0; h < s.Hkv; ++h) {
      if (rowcut) {
        const int64_t R = (int64_t)n * G;
        for (int64_t k = 0; k < R; k += kPrefillRows) {
          const int32_t ft = (int32_t)(k / G), lt = (int32_t)((std::min<int64_t>(R, k + kPrefillRows) - 1) / G);
          tiles.push_back(Item{i, h, cu[i] + ft, pack_ntok(lt - ft + 1, (int32_t)(k - (int64_t)ft * G)),
                               L[i] - n + ft, 0, L[i] - n + lt + 1, -1});
          tile_key.push_back((int64_t)i * s.Hkv + h);
        }
        continue;
      }
      for (int32_t r0 = 0; r0 < n; r0 += tpt) {
        const int32_t r1 = std::min(n, r0 + tpt);
        tiles.push_back(Item{i, h, cu[i] + r0, r1 - r0, L[i] - n + r0, 0, L[i] - n + r1, -1});
        tile_key.push_back((int64_t)i * s.Hkv + h);
      }
    }
  }
  for (size_t k = 0; k < tiles.size();) {
    const bool sib = k + 1 < tiles.size() && tile_key[k + 1] == tile_key[k];
    const size_t kn = sib ? k + 2 : k + 1;
    int64_t steps = 0;
    for (size_t u = k; u < kn; ++u) steps = std::max<int64_t>(steps, cdiv(tiles[u].kend, kPrefillKeys));
    int64_t parts = f32 ? 1 : cdiv(steps, fair);
    if (steps <= fair + fair / 2) parts = 1;
    const int64_t per = cdiv(steps, std::max<int64_t>(parts, 1)) * kPrefillKeys;
    for (size_t u = k; u < kn; ++u) {
      const Item &t = tiles[u];
      const int64_t tparts = parts <= 1 ? 1 : cdiv(t.kend, per);
      if (tparts <= 1) {
        pre.push_back(t);
        pre_key.push_back(tile_key[u]);
        continue;
      }
      for (int32_t tk = t.tok0; tk < t.tok0 + item_ntok(t); ++tk) nsplit[tk] = (int32_t)tparts;
      for (int64_t pc = 0; pc < tparts; ++pc) {
        Item piece = t;
        piece.kbeg = (int32_t)(pc * per);
        piece.kend = (int32_t)std::min<int64_t>(t.kend, (pc + 1) * per);
        piece.split = (int32_t)pc;
        pre.push_back(piece);
        pre_key.push_back(tile_key[u]);
      }
    }
    k = kn;
  }

  // level tiles: each level's members stacked against the keys it adds.  One
  // chunk length for all levels, sized so the levels give about kPrefillSlots
  // tiles in all (chunks of at least 256 keys); a member's partials are numbered
  // along its path from the top level down, then its tail.
  std::vector<int32_t> lev_npc(nlev, 0), lev_off(nlev, 0), lev_tok(nlev, 0);
  {
    int64_t work = 0;
    for (int32_t g = 0; g < nlev; ++g) {
      const CascNode &nd = p.tree[g];
      lev_tok[g] = (int32_t)p.toklist.size();
      for (int32_t j : nd.members)
        for (int32_t t = cu[j]; t < cu[j + 1]; ++t) p.toklist.push_back(t);
      const int32_t nt = (int32_t)p.toklist.size() - lev_tok[g];
      const int32_t base = nd.parent >= 0 ? p.tree[nd.parent].prefix : 0;
      work += cdiv(nt, tpt) * s.Hkv * (int64_t)(nd.prefix - base);
    }
    const int64_t lchunk = std::max<int64_t>(256, round_up(cdiv(work, kPrefillSlots), kPrefillKeys));
    for (int32_t g = 0; g < nlev; ++g) {
      const CascNode &nd = p.tree[g];
      const int32_t base = nd.parent >= 0 ? p.tree[nd.parent].prefix : 0;
      const int32_t seg = nd.prefix - base;
      int64_t npc = cdiv(seg, lchunk);
      const int32_t pchunk = (int32_t)round_up(cdiv(seg, npc), kPrefillKeys);
      npc = cdiv(seg, pchunk);
      lev_npc[g] = (int32_t)npc;
      lev_off[g] = nd.parent >= 0 ? lev_off[nd.parent] + lev_npc[nd.parent] : 0;
      const int32_t off = lev_tok[g];
      const int32_t nt = (g + 1 < nlev ? lev_tok[g + 1] : (int32_t)p.toklist.size()) - off;
      const int32_t ntile = (int32_t)cdiv(nt, tpt);
      for (int32_t h = 0; h < s.Hkv; ++h)
        for (int32_t tl = 0; tl < ntile; ++tl)
          for (int32_t c = 0; c < npc; ++c) {
            const int32_t a = tl * tpt, b = std::min(nt, a + tpt);
            pre.push_back(Item{nd.members[0], h, off + a, b - a, -1, base + c * pchunk,
                               std::min(nd.prefix, base + (c + 1) * pchunk), lev_off[g] + c});
            pre_key.push_back(((int64_t)batch + g) * s.Hkv + h);
            ++p.n_cascade_items;
          }
    }
  }

  // split-KV chunk: one length for the batch, sized for ~split_target items.
  // When MFMA tiles share the launch, the chunks run beside them, so a chunk
  // only has to finish within the tiles' estimated duration: stretch it to what
  // one wavefront streams in that time (fewer partials to merge).
  int64_t dec_keys = 0;
  for (int32_t i = 0; i < batch; ++i) {
    if (!is_decode(i)) continue;
    dec_keys += (int64_t)(L[i] - own_from(i)) * s.Hkv;
  }
  int64_t chunk64 =
      std::max<int64_t>(s.split_min_keys, round_up(cdiv(dec_keys, s.split_target), kDecodeKeys));
  if (!f32 && !pre.empty()) {
    int64_t longest = 0, steps_all = 0;
    for (const Item &it : pre) {
      const int64_t st = item_work(it);
      longest = std::max(longest, st);
      steps_all += st;
    }
    const int64_t est_steps = std::max(longest, cdiv(steps_all, kPrefillSlots));
    chunk64 = std::max(chunk64, round_up(est_steps * kConcurrentKeysPerStep, kDecodeKeys));
    // When no tile writes partials and every decode's range is within half a
    // chunk more than that, one chunk per request: the merge launch would
    // otherwise run for a handful of tokens.
    bool tile_partials = nlev > 0;
    for (const Item &it : pre) tile_partials |= it.split >= 0;
    int64_t dmax = 0;
    for (int32_t i = 0; i < batch; ++i)
      if (is_decode(i)) dmax = std::max<int64_t>(dmax, L[i] - own_from(i));
    if (!tile_partials && dmax > chunk64 && 2 * dmax <= 3 * chunk64)
      chunk64 = round_up(dmax, kDecodeKeys);
  }
  const int32_t chunk = (int32_t)std::min<int64_t>(chunk64, 1 << 30);
  p.decode_chunk = chunk;

  // Split-KV items.  Longest first (the launch runs them in order): every full
  // chunk has the longest length, so those go out in generation order and only
  // the shorter last chunks (one per request and KV head) are sorted.  Written
  // through raw pointers into vectors sized up front.
  {
    int64_t nfull = 0, nlast = 0;
    for (int32_t i = 0; i < batch; ++i) {
      if (!is_decode(i)) continue;
      const int32_t keys = L[i] - own_from(i);
      nfull += (int64_t)(keys / chunk) * s.Hkv;
      nlast += keys % chunk ? s.Hkv : 0;
    }
    std::vector<Item> &last = p.tmp.dlast;
    dec.resize(nfull);
    last.resize(nlast);
    Item *wf = dec.data(), *wl = last.data();
    const int32_t Hkv = s.Hkv;
    for (int32_t i = 0; i < batch; ++i) {
      if (!is_decode(i)) continue;
      const int32_t g = deepest[i];
      // outside any cascade: all keys, partials 0..; else the keys past the
      // deepest level, partials after that level's
      const int32_t from = g >= 0 ? p.tree[g].prefix : 0;
      const int32_t first = g >= 0 ? lev_off[g] + lev_npc[g] : 0;
      const int32_t n = n_of(i), Li = L[i], c0 = cu[i];
      const int32_t ns = (int32_t)cdiv(Li - from, chunk);
      for (int32_t t = c0; t < cu[i + 1]; ++t) nsplit[t] = first + ns;
      const bool single = g < 0 && ns == 1;  // the whole range in one item: final output
      // KV heads innermost: the heads of one chunk read interleaved rows of the
      // same pages at about the same time
      for (int32_t c = 0; c < ns; ++c) {
        const int32_t kb = from + c * chunk, ke = std::min(Li, kb + chunk);
        Item *&w = ke - kb == chunk ? wf : wl;
        for (int32_t h = 0; h < Hkv; ++h)
          *w++ = Item{i, h, c0, n, Li - n, kb, ke, single ? -1 : first + c};
      }
      if (g >= 0) ++p.cascade_members;
    }
    // the shorter chunks come in runs of Hkv (one per request): order the runs
    const int64_t nruns = nlast / Hkv;
    std::vector<int32_t> &ro = p.tmp.runs;
    ro.resize(nruns);
    std::iota(ro.begin(), ro.end(), 0);
    std::stable_sort(ro.begin(), ro.end(), [&](int32_t x, int32_t y) {
      return (last[(int64_t)x * Hkv].kend - last[(int64_t)x * Hkv].kbeg) >
             (last[(int64_t)y * Hkv].kend - last[(int64_t)y * Hkv].kbeg);
    });
    dec.resize(nfull + nlast);
    Item *w = dec.data() + nfull;
    for (int32_t r : ro)
      for (int32_t h = 0; h < Hkv; ++h) *w++ = last[(int64_t)r * Hkv + h];
  }

  // partials and merge list
  p.tok_pbase.assign(T, -1);
  int64_t np = 0;
  for (int32_t t = 0; t < T; ++t)
    if (nsplit[t] >= 2) {
      p.tok_pbase[t] = (int32_t)np;
      p.merge.push_back(t);
      p.merge.push_back((int32_t)np);
      p.merge.push_back(nsplit[t]);
      np += nsplit[t];
    }
  if (np > INT32_MAX) {
    *msg = "too many partial results";
    return RPKV_ERR_CAPACITY;
  }
  p.n_partials = np;

  // launch order
  p.n_prefill_real = (int32_t)pre.size();
  if (f32) {
    std::stable_sort(pre.begin(), pre.end(),
                     [](const Item &a, const Item &b) { return item_work(a) > item_work(b); });
    std::swap(p.prefill, pre);
    p.tiles_per_block = 1;
  } else {
    // tiles per workgroup: pairs in ping-pong pay off once tiles are long (and
    // pages hold >= 16 keys: the pair body for smaller pages spills registers)
    int tpb = s.tiles_per_block;
    if (tpb == 0 && s.P < 16) tpb = 1;
    if (tpb == 0) {
      int64_t steps = 0;
      for (const Item &it : pre) steps += item_work(it);
      tpb = !pre.empty() && steps >= (int64_t)kPairMinSteps * (int64_t)pre.size() ? 2 : 1;
    }
    p.tiles_per_block = tpb;
    Item pad{};
    std::vector<int64_t> &work = p.tmp.work;
    std::vector<int32_t> &order = p.tmp.order;
    if (tpb == 1) {
      work.resize(pre.size());
      for (size_t k = 0; k < pre.size(); ++k) work[k] = item_work(pre[k]);
      xcd_order(work, pre_key, 1, &order);
      p.prefill.resize(order.size());
      for (size_t b = 0; b < order.size(); ++b) p.prefill[b] = order[b] >= 0 ? pre[order[b]] : pad;
    } else {
      // Workgroups of two sibling items sharing one K/V stream: the same
      // request (or cascade level) and KV head, the same first key, and for
      // cascade level tiles the same last key; consecutive row blocks pair up,
      // an unpaired item runs with an empty partner.  The units are ordered like
      // single items, by the longer of the two ranges.
      std::vector<int32_t> &idx = p.tmp.idx;
      idx.resize(pre.size());
      std::iota(idx.begin(), idx.end(), 0);
      auto unit_of = [&](int32_t k) {
        const Item &it = pre[k];
        const bool casc = it.pos0 < 0;
        return std::make_tuple(pre_key[k], casc, it.kbeg, casc ? it.kend : 0);
      };
      std::sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
        const auto ux = unit_of(x), uy = unit_of(y);
        return ux != uy ? ux < uy : pre[x].tok0 < pre[y].tok0;
      });
      std::vector<int32_t> &second = p.tmp.second;
      std::vector<int64_t> &ukey = p.tmp.ukey;
      std::vector<int32_t> &first = p.tmp.first;
      first.clear();
      second.clear();
      ukey.clear();
      work.clear();
      for (size_t k = 0; k < idx.size();) {
        const int32_t x = idx[k];
        const bool pair = k + 1 < idx.size() && unit_of(idx[k + 1]) == unit_of(x);
        const int32_t y = pair ? idx[k + 1] : -1;
        first.push_back(x);
        second.push_back(y);
        ukey.push_back(pre_key[x]);
        const int32_t kend = pair ? std::max(pre[x].kend, pre[y].kend) : pre[x].kend;
        work.push_back(cdiv(std::max(kend - pre[x].kbeg, 1), kPrefillKeys));
        k += pair ? 2 : 1;
      }
      xcd_order(work, ukey, 1, &order);
      p.prefill.resize(2 * order.size());
      for (size_t b = 0; b < order.size(); ++b) {
        const int32_t u = order[b];
        p.prefill[2 * b] = u >= 0 ? pre[first[u]] : pad;
        p.prefill[2 * b + 1] = u >= 0 && second[u] >= 0 ? pre[second[u]] : pad;
      }
    }
  }
  std::swap(p.decode, dec);
  p.plan_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_start)
                  .count();
  return RPKV_OK;
}

}  // namespace rpkv
