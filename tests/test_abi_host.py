"""Host-side tests of the C ABI (no GPU): the library loads and exports every
function the header declares, capability checks, validation errors, and the
planner's work partition covers every visible (token, head, key) exactly once."""
import ctypes
import os
import re

import numpy as np
import pytest

from tests import _golden
from workloads import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def rp():
    import ragged_paged_kv_store_amd as rp
    return rp


def header_functions():
    text = open(os.path.join(ROOT, "include", "rpkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rpkv_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(rp):
    declared = header_functions()
    assert len(declared) >= 15
    lib = ctypes.CDLL(rp.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(rp.EXPORTS) == declared


def test_status_strings(rp):
    for code, name in rp.STATUS.items():
        assert rp.lib.rpkv_status_string(code).decode() == name


BASE = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=0, max_batch=64,
            num_pages=1024, max_tokens=8192, max_pages_per_req=512)


@pytest.mark.parametrize("change,ok", [
    ({}, True),
    (dict(head_dim=64), False),             # bf16 kernels are built for 128
    (dict(dtype=1, head_dim=64), True),
    (dict(dtype=1, head_dim=96), False),
    (dict(num_q_heads=30), False),          # Hq % Hkv
    (dict(page_size=12), False),            # not a power of two
    (dict(page_size=1), True),
    (dict(num_kv_heads=32), True),          # MHA
    (dict(num_kv_heads=1), True),           # G = 32
    (dict(num_q_heads=128, num_kv_heads=1), True),   # G = 128, the largest
    (dict(num_q_heads=256, num_kv_heads=1), False),
    (dict(dtype=1, num_kv_heads=1), False),           # fp32 tiles hold 16 rows: G <= 16
    (dict(dtype=1, num_q_heads=16, num_kv_heads=1), True),
    (dict(dtype=7), False),
    (dict(decode_max_rows=17), False),
])
def test_supports(rp, change, ok):
    got, msg = rp.supports(**{**BASE, **change})
    assert got == ok, msg


def make_plan(rp, spec, **kw):
    return rp.Plan(num_q_heads=spec.Hq, num_kv_heads=spec.Hkv, head_dim=spec.D,
                   page_size=spec.P, dtype=0 if spec.dtype == "bf16" else 1,
                   max_batch=max(spec.bs, 1), num_pages=spec.num_pages,
                   max_tokens=max(spec.T, 1), max_pages_per_req=spec.page_table.shape[1], **kw)


@pytest.mark.parametrize("batch,P,stride,cols,null", [
    (-1, 16, 8, 8, None), (2, 12, 8, 8, None), (2, 16, 4, 8, None), (2, 16, 8, -1, None),
    (2, 16, 8, 8, "n"), (2, 16, 8, 8, "counts"),
])
def test_build_metadata_rejects_bad_arguments(rp, batch, P, stride, cols, null):
    """Checked on the host before anything is enqueued (no GPU needed)."""
    fake = ctypes.c_void_p(0x1000)
    args = {k: fake for k in ("nc", "n", "bt", "qsl", "seq", "pos", "slots", "lg", "counts")}
    if null:
        args[null] = None
    st = rp.lib.rpkv_build_metadata(batch, args["nc"], args["n"], None, args["bt"], stride, cols, P,
                                    16, args["qsl"], args["seq"], args["pos"], args["slots"],
                                    args["lg"], args["counts"], None)
    assert st == 1, rp.lib.rpkv_last_error()


def test_last_indices_worked_example(rp):
    g = _golden.load("p1_worked_example.txt")
    p = rp.Plan(num_q_heads=16, num_kv_heads=8, head_dim=128, page_size=1, dtype=0, max_batch=3,
                num_pages=64, max_tokens=16, max_pages_per_req=9)
    p.plan_host(g["cu_seqlens_q"], g["cache_seqlens"], 9, np.array(g["page_table_cut"]))
    assert p.last_indices().tolist() == g["last_indices"]
    # a request with no queries gets -1
    p.plan_host([0, 2, 2, 3], [4, 5, 6], 9)
    assert p.last_indices().tolist() == [1, -1, 2]


@pytest.mark.parametrize("cu,L,cols,pt,status", [
    ([1, 2], [2], 2, None, 1),          # cu[0] != 0
    ([0, 3, 2], [3, 3], 2, None, 1),    # decreasing
    ([0, 4], [3], 2, None, 1),          # n > L
    ([0, 1], [40], 2, None, 1),         # needs 3 columns of 16
    ([0, 1], [4], 2, [[5000, 0]], 1),   # page id out of range (host table given)
    ([0, 1], [4], 2, [[-1, 0]], 1),     # negative page id
])
def test_invalid_batches_rejected(rp, cu, L, cols, pt, status):
    p = rp.Plan(**BASE)
    with pytest.raises(rp.RpkvError) as e:
        p.plan_host(cu, L, cols, None if pt is None else np.array(pt))
    assert e.value.status == status


def test_capacity_errors(rp):
    p = rp.Plan(**{**BASE, "max_batch": 2, "max_tokens": 4})
    with pytest.raises(rp.RpkvError) as e:
        p.plan_host([0, 1, 2, 3], [1, 1, 1], 1)
    assert e.value.status == 6
    with pytest.raises(rp.RpkvError) as e:
        p.plan_host([0, 5], [5], 1)
    assert e.value.status == 6


def test_not_prepared_errors(rp):
    p = rp.Plan(**BASE)
    with pytest.raises(rp.RpkvError) as e:
        p.info()
    assert e.value.status == 4
    st = rp.lib.rpkv_attend(p._h, None, None, None, None, 0.1, None)
    assert st == 4


def test_cascade_hint_checked_against_host_table(rp):
    p = rp.Plan(**BASE)
    pt = np.array([[1, 2, 3], [1, 2, 4], [1, 9, 5]], np.int32)
    p.plan_host([0, 1, 2, 3], [40, 40, 40], 3, pt, groups=[(0, 2, 32)])
    with pytest.raises(rp.RpkvError):
        p.plan_host([0, 1, 2, 3], [40, 40, 40], 3, pt, groups=[(0, 3, 32)])
    with pytest.raises(rp.RpkvError):   # not a multiple of the page size
        p.plan_host([0, 1, 2, 3], [40, 40, 40], 3, pt, groups=[(0, 2, 20)])
    with pytest.raises(rp.RpkvError):   # overlapping groups
        p.plan_host([0, 1, 2, 3], [40, 40, 40], 3, pt, groups=[(0, 2, 16), (1, 2, 16)])
    # nested groups form two levels
    pt = np.array([[1, 2, 3], [1, 2, 4], [1, 9, 5]], np.int32)
    p.plan_host([0, 1, 2, 3], [40, 40, 40], 3, pt, groups=[(0, 3, 16), (0, 2, 32)])
    assert p.cascade_tree() == [{"members": (0, 1, 2), "prefix": 16, "parent": -1},
                                {"members": (0, 1), "prefix": 32, "parent": 0}]
    assert p.info()["cascade_depth"] == 2
    with pytest.raises(rp.RpkvError):   # nested without a longer prefix
        p.plan_host([0, 1, 2, 3], [40, 40, 40], 3, pt, groups=[(0, 3, 16), (0, 2, 16)])
    with pytest.raises(rp.RpkvError):   # nested level's pages differ
        p.plan_host([0, 1, 2, 3], [40, 40, 40], 3, pt, groups=[(0, 3, 16), (1, 2, 32)])


# ------------------------------------------------------------------ coverage

def check_coverage(rp, plan, spec):
    """Every visible (token, q head, key) is covered by exactly one item, split
    numbers of a (token, head) are -1 alone or exactly 0..S-1, cascade tiles only
    cover keys every row can see, and key ranges never pass L."""
    G = spec.G
    cu = spec.cu_q
    tok_req = np.repeat(np.arange(spec.bs), spec.n)
    tl = plan.token_list()
    cover = {}
    for kind in (0, 1):
        for it in plan.items(kind):
            req, kvh, tok0, nfield, pos0, kbeg, kend, split = [int(x) for x in it]
            # token count, and the rows of the first token before the tile
            ntok, row0 = nfield & 0xFFFF, (nfield >> 16) & 0xFF
            if ntok == 0:
                continue
            assert 0 <= kbeg < kend
            cap = 16 if kind == 1 or spec.dtype != "bf16" else 128
            if row0 or ntok * G > cap:
                # rows cut every 128 inside a token: only for unsplit bf16 tiles
                # with G not dividing 128, every cut at a multiple of 128 rows
                assert kind == 0 and spec.dtype == "bf16" and 128 % G and split == -1 and pos0 >= 0
                assert 0 <= row0 < G and (tok0 - int(cu[req])) * G + row0 == \
                    ((tok0 - int(cu[req])) * G + row0) // 128 * 128
                last_row = (tok0 - int(cu[req])) * G + row0 + min(cap, ntok * G - row0)
                assert last_row % 128 == 0 or last_row == int(spec.n[req]) * G
                assert (ntok - 1) * G < row0 + cap
            else:
                assert ntok * G <= cap or ntok == 1
            rows = min(cap, ntok * G - row0) if kind == 0 else ntok * G
            heads_of = {}
            for j in range(row0, row0 + rows):
                heads_of.setdefault(j // G, []).append(j % G)
            for r in range(ntok):
                if pos0 < 0:
                    t = int(tl[tok0 + r])
                else:
                    t = tok0 + r
                i = int(tok_req[t])
                a = int(spec.L[i]) - int(spec.n[i]) + (t - int(cu[i]))
                if pos0 >= 0:
                    assert i == req and pos0 + r == a
                    hi = min(kend, a + 1)
                else:
                    assert kend - 1 <= a, "cascade tile covers a key a row cannot see"
                    # the tile reads request `req`'s pages: every row's request
                    # must hold the same pages for those keys
                    pk = np.arange(kbeg // spec.P, (kend - 1) // spec.P + 1)
                    assert (spec.page_table[req, pk] == spec.page_table[i, pk]).all(), \
                        "cascade tile reads pages a row's request does not share"
                    hi = kend
                assert kend <= int(spec.L[i]) or pos0 < 0
                for g in heads_of[r]:
                    h = kvh * G + g
                    cover.setdefault((t, h), []).append((kbeg, hi, split))
    for t in range(spec.T):
        i = int(tok_req[t])
        a = int(spec.L[i]) - int(spec.n[i]) + (t - int(cu[i]))
        for h in range(spec.Hq):
            segs = sorted(cover.get((t, h), []))
            assert segs, (t, h)
            pos = 0
            for lo, hi, _ in segs:
                if hi <= lo:
                    continue
                assert lo == pos, (t, h, segs)
                pos = hi
            assert pos == a + 1, (t, h, segs)
            splits = sorted(s for _, _, s in segs)
            assert splits == [-1] or splits == list(range(len(segs))), (t, h, splits)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_small_configs_covered_exactly_once(rp, cid):
    spec = synth.small_config(cid)
    p = make_plan(rp, spec)
    p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table, spec.groups)
    check_coverage(rp, p, spec)
    if spec.groups:
        assert p.info()["cascade_members"] == spec.groups[0][1]


@pytest.mark.parametrize("tpb", [0, 1, 2])
@pytest.mark.parametrize("Hq,Hkv,n,L", [
    (64, 1, [5, 1, 2], [300, 700, 41]),      # 2 tokens x 64 heads per tile
    (128, 1, [3, 1, 1], [600, 257, 1]),      # 1 token x 128 heads per tile
    (128, 2, [1, 1, 1], [100, 2000, 5000]),  # decodes of 64 rows run as tiles
])
def test_largest_groups_covered_exactly_once(rp, Hq, Hkv, n, L, tpb):
    spec = synth.build("bigG", "bf16", Hq, Hkv, 128, 16, n, L, 7, np.random.default_rng(Hq + Hkv), 1.3)
    p = make_plan(rp, spec, tiles_per_block=tpb)
    p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table)
    check_coverage(rp, p, spec)
    assert len(p.items(1)) == 0, "n * G > 16: no split-KV items"


@pytest.mark.parametrize("seed", range(12))
def test_random_batches_covered_exactly_once(rp, seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 2, 4, 7, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4]))
    P = int(rng.choice([1, 4, 16, 64]))
    bs = int(rng.integers(1, 12))
    n, L = [], []
    for _ in range(bs):
        kind = rng.integers(0, 4)
        if kind == 0:
            x = int(rng.integers(1, 300)); n.append(x); L.append(x)
        elif kind == 1:
            L.append(int(rng.integers(1, 3000))); n.append(1)
        elif kind == 2:
            l = int(rng.integers(2, 2000)); L.append(l); n.append(int(rng.integers(1, min(l, 3) + 1)))
        else:
            L.append(int(rng.integers(0, 50))); n.append(0)
    dtype = "bf16" if seed % 3 else "f32"
    spec = synth.build("r", dtype, G * Hkv, Hkv, 128, P, n, L, seed, np.random.default_rng(seed), 1.2)
    kw = dict(split_min_keys=int(rng.choice([0, 32, 64])), split_target=int(rng.choice([0, 64])))
    kw["tiles_per_block"] = int(rng.choice([0, 1, 2]))
    p = make_plan(rp, spec, **kw)
    p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table)
    check_coverage(rp, p, spec)
    if dtype == "bf16" and kw["tiles_per_block"]:
        assert p.info()["tiles_per_block"] == kw["tiles_per_block"]
        assert len(p.items(0)) % (8 * kw["tiles_per_block"]) == 0
    if p.info()["tiles_per_block"] == 2:
        check_sibling_pairs(p)


def test_full_config_plans(rp):
    """The five full-size batches plan; their partitions are exactly-once (C2,
    C4 checked fully; C3/C5 by counts) and the planner is fast."""
    for cid in (2, 4):
        spec = synth.full_config(cid)
        p = make_plan(rp, spec)
        p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table, spec.groups)
        check_coverage(rp, p, spec)
    spec = synth.full_config(5)
    p = make_plan(rp, spec)
    p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table, spec.groups)
    info = p.info()
    assert info["cascade_members"] == 64 and info["num_cascade_items"] > 0
    assert info["plan_host_us"] < 50_000


def check_sibling_pairs(plan):
    """With two tiles per workgroup, the tiles of a workgroup share one K/V
    stream: the second (when present) has the first's request, KV head and
    first key (and, for cascade level tiles, last key); padding never comes
    first."""
    items = plan.items(0)
    assert len(items) % 16 == 0
    for p in range(len(items) // 2):
        a, b = items[2 * p], items[2 * p + 1]
        if b[3] == 0:
            continue
        assert a[3] > 0, p
        assert (a[0], a[1], a[5]) == (b[0], b[1], b[5]), (p, a, b)
        assert (a[4] < 0) == (b[4] < 0), (p, a, b)
        if a[4] < 0:
            assert a[6] == b[6], (p, a, b)


def test_tiles_per_block_choice_and_pair_layout(rp):
    """The planner runs MFMA tiles in pairs (two per 8-wavefront workgroup, in
    ping-pong) when the batch's tiles average at least 24 steps of 64 keys, else
    one per 4-wavefront workgroup; the shape can force either.  Either layout
    covers every visible (token, head, key) exactly once, and the list is padded
    to whole workgroups on all 8 XCDs."""
    for cid, want in ((2, 1), (4, 2), (5, 2)):
        spec = synth.full_config(cid)
        p = make_plan(rp, spec)
        p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table, spec.groups)
        assert p.info()["tiles_per_block"] == want, cid
        if want == 2:
            check_sibling_pairs(p)
    for cid in (2, 4):
        spec = synth.small_config(cid)
        for tpb in (1, 2):
            p = make_plan(rp, spec, tiles_per_block=tpb)
            p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table, spec.groups)
            assert p.info()["tiles_per_block"] == tpb
            assert len(p.items(0)) % (8 * tpb) == 0
            check_coverage(rp, p, spec)
            if tpb == 2:
                check_sibling_pairs(p)
    ok, _ = rp.supports(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=0,
                        max_batch=4, num_pages=64, max_tokens=64, max_pages_per_req=8,
                        tiles_per_block=3)
    assert not ok



def test_row_cut_tiles_covered_exactly_once(rp):
    """The row-cut cases of the GPU test plan tiles that start inside a token
    beside key-split whole-token tiles, in both tile arrangements, and cover
    every visible (token, head, key) exactly once."""
    from tests.test_gpu_row_cut import CASES
    for name, Hq, Hkv, n, L in CASES:
        spec = synth.build(name, "bf16", Hq, Hkv, 128, 16, n, L, 31, np.random.default_rng(0), 1.25)
        for tpb in (1, 2):
            p = make_plan(rp, spec, tiles_per_block=tpb)
            p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table)
            items = p.items(0)
            assert ((items[:, 3] >> 16) > 0).any(), name
            assert (items[:, 7] >= 0).any(), name
            check_coverage(rp, p, spec)
            if tpb == 2:
                check_sibling_pairs(p)


def test_mixed_launch_stretches_chunks_rather_than_merge_a_few_decodes(rp):
    """In a launch with MFMA tiles and no tile partials, decodes up to half a
    chunk longer than the split-KV chunk run as one chunk each (no merge launch
    for a handful of tokens); longer ones are still split."""
    def info(L_dec):
        n = [512] * 4 + [1] * len(L_dec)
        L = [4608] * 4 + list(L_dec)
        spec = synth.build("stretch", "bf16", 28, 4, 128, 16, n, L, 3, np.random.default_rng(0), 1.25)
        p = make_plan(rp, spec)
        p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table)
        check_coverage(rp, p, spec)
        return p.info()
    base = info([300, 500])
    chunk = base["decode_chunk"]
    assert base["num_partials"] == 0 and base["num_prefill_items"] > 0
    for L in (chunk + 40, chunk * 3 // 2 - 32):
        i = info([300, L])
        assert i["num_partials"] == 0 and i["decode_chunk"] >= L, (L, i)
    i = info([300, chunk * 3 // 2 + 64])
    assert i["num_partials"] == 2 and i["decode_chunk"] == chunk
