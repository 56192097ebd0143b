// Host-only driver of the planner for sanitizer builds (AddressSanitizer and
// UndefinedBehaviorSanitizer): compiled with g++ together with csrc/plan.cpp,
// no HIP.  It plans seeded random batches -- prefill, chunked-prefill, decode,
// speculative and empty requests; bf16 and fp32; page sizes 1..64; GQA 1..16;
// shared-prefix trees found in the page table or given as nested hints -- and
// checks each work partition:
//  * every visible (token, query head, key) is covered exactly once, and a
//    (token, head) has either one final item or partials numbered 0..S-1 whose
//    count matches its merge record;
//  * a cascade tile only covers keys all its rows see, through pages every
//    row's request shares;
//  * the partition fits the plan's metadata capacity;
// and checks find_bad_slot against a brute-force scan.  Exit status 0 = clean.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "rpkv_internal.h"

namespace {

struct Rng {  // splitmix64
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int64_t in(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
};

int g_fail = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);         \
      std::fprintf(stderr, "\n");                \
      ++g_fail;                                  \
      return false;                              \
    }                                            \
  } while (0)

struct Batch {
  int32_t Hq, Hkv, P, dtype, cols;
  std::vector<int32_t> cu, L, pt;  // pt [bs, cols]
  std::vector<rpkv_prefix_group> groups;
  int32_t detect = 0;
  int32_t bs() const { return (int32_t)L.size(); }
};

bool check_partition(const Batch &b, const rpkv::Shape &s, const rpkv::HostPlan &hp) {
  const int32_t G = s.G(), bs = b.bs();
  const int32_t T = b.cu[bs];
  std::vector<int32_t> req_of(T), a_of(T);
  for (int32_t i = 0; i < bs; ++i)
    for (int32_t t = b.cu[i]; t < b.cu[i + 1]; ++t) {
      req_of[t] = i;
      a_of[t] = b.L[i] - (b.cu[i + 1] - b.cu[i]) + (t - b.cu[i]);
    }
  // per (token, head): (kbeg, hi, split)
  std::vector<std::vector<std::tuple<int32_t, int32_t, int32_t>>> seg((size_t)T * s.Hq);
  auto visit = [&](const rpkv::Item &it, bool decode) -> bool {
    if (it.ntok == 0) return true;
    CHECK(0 <= it.kbeg && it.kbeg < it.kend, "empty or negative key range");
    CHECK(it.kvh >= 0 && it.kvh < s.Hkv, "bad KV head");
    // a tile's rows: a run of its tokens' (token, head) rows from row0 on
    const int32_t ntok = rpkv::item_ntok(it), row0 = rpkv::item_row0(it);
    const int32_t cap = decode ? rpkv::kDecodeRows
                               : (s.dtype == RPKV_F32 ? rpkv::kF32Rows : rpkv::kPrefillRows);
    CHECK(ntok > 0 && row0 >= 0 && row0 < G, "token count %d, row offset %d", ntok, row0);
    if (decode) CHECK(ntok * G <= cap && row0 == 0, "decode item of %d rows", ntok * G);
    if (row0 > 0 || ntok * G > cap) {
      // cut every 128 rows inside a token: unsplit bf16 tiles, G not dividing 128
      CHECK(!decode && s.dtype == RPKV_BF16 && rpkv::kPrefillRows % G != 0 && it.split < 0 &&
                it.pos0 >= 0,
            "row-cut item that may not be cut");
      const int64_t first = (int64_t)(it.tok0 - b.cu[it.req]) * G + row0;
      const int64_t last = first + rpkv::item_rows(it, G, cap);
      const int64_t R = (int64_t)(b.cu[it.req + 1] - b.cu[it.req]) * G;
      CHECK(first % cap == 0 && (last % cap == 0 || last == R), "row cut at %lld..%lld",
            (long long)first, (long long)last);
      CHECK((ntok - 1) * G < row0 + cap, "tile of %d tokens from row %d", ntok, row0);
    } else {
      CHECK(ntok * G <= cap || ntok == 1, "tile of %d rows", ntok * G);
    }
    const int32_t nrows = decode ? ntok * G : rpkv::item_rows(it, G, ntok == 1 ? ntok * G : cap);
    for (int32_t r = 0; r < ntok; ++r) {
      int32_t t, hi;
      if (it.pos0 < 0) {
        CHECK(it.tok0 + r < (int32_t)hp.toklist.size(), "token list index");
        t = hp.toklist[it.tok0 + r];
        CHECK(t >= 0 && t < T, "token list entry");
        CHECK(it.kend - 1 <= a_of[t], "cascade tile covers a key a row cannot see");
        const int32_t i = req_of[t];
        for (int32_t pg = it.kbeg / b.P; pg <= (it.kend - 1) / b.P; ++pg)
          CHECK(b.pt[(size_t)it.req * b.cols + pg] == b.pt[(size_t)i * b.cols + pg],
                "cascade tile reads a page request %d does not share", i);
        hi = it.kend;
      } else {
        t = it.tok0 + r;
        CHECK(t < T && req_of[t] == it.req && it.pos0 + r == a_of[t], "tile row position");
        CHECK(it.kend <= b.L[it.req], "key range past L");
        hi = std::min(it.kend, a_of[t] + 1);
      }
      for (int32_t g = 0; g < G; ++g) {
        const int32_t j = r * G + g - row0;  // row of the tile
        if (j < 0 || j >= nrows) continue;
        seg[(size_t)t * s.Hq + it.kvh * G + g].emplace_back(it.kbeg, hi, it.split);
      }
    }
    return true;
  };
  for (const rpkv::Item &it : hp.prefill)
    if (!visit(it, false)) return false;
  for (const rpkv::Item &it : hp.decode)
    if (!visit(it, true)) return false;
  std::map<int32_t, int32_t> merge_count;
  for (size_t m = 0; m + 2 < hp.merge.size(); m += 3) merge_count[hp.merge[m]] = hp.merge[m + 2];
  for (int32_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < s.Hq; ++h) {
      auto &v = seg[(size_t)t * s.Hq + h];
      std::sort(v.begin(), v.end());
      int32_t pos = 0;
      std::vector<int32_t> splits;
      for (auto &x : v) {
        splits.push_back(std::get<2>(x));
        if (std::get<1>(x) <= std::get<0>(x)) continue;
        CHECK(std::get<0>(x) == pos, "token %d head %d: gap or overlap at key %d", t, h, pos);
        pos = std::get<1>(x);
      }
      CHECK(pos == a_of[t] + 1, "token %d head %d covers %d of %d keys", t, h, pos, a_of[t] + 1);
      std::sort(splits.begin(), splits.end());
      if (splits.size() == 1 && splits[0] == -1) {
        CHECK(hp.tok_pbase[t] < 0, "token %d: final item but a partial base", t);
      } else {
        for (size_t k = 0; k < splits.size(); ++k)
          CHECK(splits[k] == (int32_t)k, "token %d head %d: split numbers", t, h);
        CHECK(hp.tok_pbase[t] >= 0 && merge_count[t] == (int32_t)splits.size(),
              "token %d: merge record", t);
      }
    }
  // two tiles per workgroup: siblings sharing one K/V stream, padding never first
  if (hp.tiles_per_block == 2) {
    CHECK(hp.prefill.size() % 16 == 0, "pair list not a whole number of XCD rounds");
    for (size_t k = 0; k + 1 < hp.prefill.size(); k += 2) {
      const rpkv::Item &x = hp.prefill[k], &y = hp.prefill[k + 1];
      if (y.ntok == 0) continue;
      CHECK(x.ntok > 0, "workgroup %zu: padding before a tile", k / 2);
      CHECK(x.req == y.req && x.kvh == y.kvh && x.kbeg == y.kbeg && (x.pos0 < 0) == (y.pos0 < 0) &&
                (x.pos0 >= 0 || x.kend == y.kend),
            "workgroup %zu: tiles that do not share K/V", k / 2);
    }
  }
  const rpkv::MetaLayout need = rpkv::meta_layout(rpkv::meta_counts(hp, s.max_batch));
  const rpkv::MetaLayout cap = rpkv::meta_layout(rpkv::meta_caps(s));
  CHECK(need.bytes <= cap.bytes, "metadata %zu bytes > capacity %zu", need.bytes, cap.bytes);
  return true;
}

// A random batch: a few requests of each kind, page ids from a small alphabet
// with copied prefixes (accidental and deliberate sharing).
Batch random_batch(Rng &rng, bool hints) {
  Batch b;
  const int32_t Gs[] = {1, 2, 4, 7, 8, 16};
  const int32_t G = Gs[rng.in(0, 5)];
  b.Hkv = (int32_t)rng.in(1, 3);
  b.Hq = G * b.Hkv;
  b.dtype = rng.in(0, 3) == 0 ? RPKV_F32 : RPKV_BF16;
  const int32_t Ps[] = {1, 2, 4, 16, 64};
  b.P = Ps[rng.in(0, 4)];
  const int32_t bs = (int32_t)rng.in(1, 14);
  std::vector<int32_t> n(bs);
  b.L.resize(bs);
  for (int32_t i = 0; i < bs; ++i) {
    switch (rng.in(0, 4)) {
      case 0: n[i] = (int32_t)rng.in(1, 200); b.L[i] = n[i]; break;            // prefill
      case 1: n[i] = (int32_t)rng.in(1, 90); b.L[i] = n[i] + (int32_t)rng.in(0, 400); break;
      case 2: n[i] = 1; b.L[i] = (int32_t)rng.in(1, 700); break;               // decode
      case 3: n[i] = (int32_t)rng.in(1, 4); b.L[i] = n[i] + (int32_t)rng.in(0, 500); break;
      default: n[i] = 0; b.L[i] = (int32_t)rng.in(0, 60); break;               // empty
    }
  }
  b.cu.assign(bs + 1, 0);
  for (int32_t i = 0; i < bs; ++i) b.cu[i + 1] = b.cu[i] + n[i];
  b.cols = 1;
  for (int32_t i = 0; i < bs; ++i) b.cols = std::max<int32_t>(b.cols, (b.L[i] + b.P - 1) / b.P);
  b.pt.assign((size_t)bs * b.cols, 0);
  const int32_t alphabet = (int32_t)rng.in(2, 6);
  for (auto &x : b.pt) x = (int32_t)rng.in(0, alphabet - 1);
  for (int32_t j = 1; j < bs; ++j)
    if (rng.in(0, 9) < 7) {
      const int32_t src = (int32_t)rng.in(0, j - 1), k = (int32_t)rng.in(0, b.cols);
      for (int32_t c = 0; c < k; ++c) b.pt[(size_t)j * b.cols + c] = b.pt[(size_t)src * b.cols + c];
    }
  if (hints && bs >= 2) {
    // nested hints over requests [0, m): every member gets the same first pages
    const int32_t m = (int32_t)rng.in(2, bs);
    int32_t minL = b.L[0];
    for (int32_t j = 0; j < m; ++j) minL = std::min(minL, b.L[j]);
    const int32_t pages = minL / b.P;
    if (pages >= 1) {
      for (int32_t j = 1; j < m; ++j)
        for (int32_t c = 0; c < pages; ++c) b.pt[(size_t)j * b.cols + c] = b.pt[c];
      const int32_t p1 = (int32_t)rng.in(1, pages);
      b.groups.push_back(rpkv_prefix_group{0, m, p1 * b.P});
      if (m >= 3 && p1 < pages)
        b.groups.push_back(rpkv_prefix_group{0, m - 1, (int32_t)rng.in(p1 + 1, pages) * b.P});
    }
  } else {
    b.detect = rng.in(0, 1) ? (int32_t)rng.in(1, 3) * b.P : 0;
  }
  return b;
}

bool run_batch(const Batch &b, Rng &rng, rpkv::HostPlan *hp) {
  rpkv_shape sh{};
  sh.num_q_heads = b.Hq;
  sh.num_kv_heads = b.Hkv;
  sh.head_dim = 128;
  sh.page_size = b.P;
  sh.dtype = b.dtype;
  sh.max_batch = b.bs() + (int32_t)rng.in(0, 3);
  sh.num_pages = 64;
  sh.max_tokens = std::max(1, b.cu[b.bs()]) + (int32_t)rng.in(0, 5);
  sh.max_pages_per_req = b.cols + (int32_t)rng.in(0, 2);
  const int32_t mins[] = {0, 32, 64};
  sh.split_min_keys = mins[rng.in(0, 2)];
  sh.split_target = rng.in(0, 1) ? 64 : 0;
  sh.tiles_per_block = (int32_t)rng.in(0, 2);
  sh.prefix_detect_keys = b.detect;
  rpkv::Shape s;
  std::string msg;
  rpkv_status st = rpkv::check_shape(&sh, &s, &msg);
  if (st == RPKV_ERR_UNSUPPORTED) return true;  // fp32 with G > 16
  CHECK(st == RPKV_OK, "shape rejected: %s", msg.c_str());
  st = rpkv::plan_batch_host(s, b.bs(), b.cu.data(), b.L.data(), b.cols, b.pt.data(),
                             b.groups.empty() ? nullptr : b.groups.data(),
                             (int32_t)b.groups.size(), hp, &msg);
  CHECK(st == RPKV_OK, "plan failed: %s", msg.c_str());
  return check_partition(b, s, *hp);
}

bool slot_check_cases(Rng &rng) {
  std::vector<int64_t> scratch;
  for (int rep = 0; rep < 300; ++rep) {
    const int64_t n = rng.in(0, 60), num_slots = rng.in(1, 80);
    std::vector<int32_t> sl(n);
    for (auto &x : sl) x = (int32_t)rng.in(-3, num_slots + 2);
    // brute force: first token t whose slot is out of range or repeats an
    // earlier token's slot, in token order of the offending (later) token
    int64_t want = -1;
    for (int64_t t = 0; t < n && want < 0; ++t) {
      if (sl[t] < 0) continue;
      if (sl[t] >= num_slots) { want = t; break; }
      for (int64_t u = 0; u < t; ++u)
        if (sl[u] == sl[t]) { want = t; break; }
    }
    std::string msg;
    const int64_t got = rpkv::find_bad_slot(sl.data(), n, num_slots, &scratch, &msg);
    // out-of-range slots are reported as soon as the scan meets them, so when
    // both kinds occur only "some bad token" is guaranteed
    CHECK((got < 0) == (want < 0), "slot check disagrees: got %lld want %lld", (long long)got,
          (long long)want);
    if (got >= 0) CHECK(!msg.empty(), "slot check without a message");
  }
  return true;
}

}  // namespace

int main(int argc, char **argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 400;
  Rng rng{12345};
  rpkv::HostPlan hp;  // reused across batches, as a plan keeps its buffers
  int planned = 0;
  for (int k = 0; k < n && g_fail == 0; ++k) {
    const Batch b = random_batch(rng, k % 3 == 2);
    if (run_batch(b, rng, &hp)) ++planned;
    if (g_fail) std::fprintf(stderr, "batch %d (bs %d, G %d, P %d, dtype %d)\n", k, b.bs(),
                             b.Hq / b.Hkv, b.P, b.dtype);
  }
  if (g_fail == 0) slot_check_cases(rng);
  std::printf("plan_sanitize: %d batches, %d failures\n", planned, g_fail);
  return g_fail ? 1 : 0;
}
