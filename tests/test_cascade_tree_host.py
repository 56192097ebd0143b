"""Multi-level cascade planning on the host (no GPU): the planner's shared-prefix
levels -- detected from the page table, or given as nested hints -- equal the
oracle's tree (oracle/prefix_tree.py), and the resulting work partition covers
every visible (token, head, key) exactly once with tiles that only read pages
their rows share."""
import numpy as np
import pytest

from oracle import prefix_tree as pt
from tests.test_abi_host import check_coverage, make_plan
from workloads import synth


@pytest.fixture(scope="module")
def rp():
    import ragged_paged_kv_store_amd as rp
    return rp


def decode_type(spec):
    return [bool(n > 0 and n * spec.G <= 16) for n in spec.n]


def oracle_tree(spec, min_keys):
    return pt.prefix_tree(spec.page_table, spec.L, spec.n, spec.P, decode_type(spec), min_keys)


def plan_tree(rp, spec, groups=(), **kw):
    p = make_plan(rp, spec, **kw)
    p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table, list(groups))
    return p, p.cascade_tree()


def depth(nodes):
    d = 0
    for k in range(len(nodes)):
        c, a = 0, k
        while a >= 0:
            c, a = c + 1, nodes[a]["parent"]
        d = max(d, c)
    return d


@pytest.mark.parametrize("shuffle", [False, True])
@pytest.mark.parametrize("P", [1, 4, 16, 64])
def test_detected_tree_matches_oracle_radix(rp, P, shuffle):
    spec = synth.radix_tree_small(seed=30 + P, shuffle=shuffle, P=P)
    for mk in (1, 64, 200, 1000):
        p, got = plan_tree(rp, spec, prefix_detect_keys=mk)
        want = oracle_tree(spec, mk)
        assert pt.canonical(got) == pt.canonical(want), mk
        assert p.info()["cascade_depth"] == depth(want)
        check_coverage(rp, p, spec)
    # the unpruned tree of this workload has its three levels
    assert depth(oracle_tree(spec, 1)) == 3


def test_nested_hints_equal_detection(rp):
    """In tree order the workload's nested hints give the same levels as
    detection, and both the oracle's tree."""
    spec = synth.radix_tree_small(seed=41, shuffle=False)
    assert len(spec.groups) == 1 + 2 + 4
    p1, hinted = plan_tree(rp, spec, spec.groups)
    p2, detected = plan_tree(rp, spec, prefix_detect_keys=1)
    assert pt.canonical(hinted) == pt.canonical(detected) == pt.canonical(oracle_tree(spec, 1))
    check_coverage(rp, p1, spec)
    assert p1.info()["cascade_members"] == 16 and p1.info()["cascade_depth"] == 3
    # hints take precedence over detection; no hints and detection off: no levels
    p3, t3 = plan_tree(rp, spec, spec.groups[:1], prefix_detect_keys=1)
    assert len(t3) == 1
    p4, t4 = plan_tree(rp, spec)
    assert t4 == [] and p4.info()["cascade_members"] == 0


def test_mixed_batch_levels_skip_prefill_requests(rp):
    """Prefill-type requests never join a level; a decode whose new tokens reach
    into a shared page does not offer that page."""
    spec = synth.radix_tree_small(seed=42, shuffle=True, extra_prefills=((300, 80), (0, 64)))
    p, got = plan_tree(rp, spec, prefix_detect_keys=1)
    assert pt.canonical(got) == pt.canonical(oracle_tree(spec, 1))
    prefill_reqs = {i for i in range(spec.bs) if not decode_type(spec)[i]}
    assert prefill_reqs and all(not (set(nd["members"]) & prefill_reqs) for nd in got)
    check_coverage(rp, p, spec)


def random_shared_batch(seed):
    """Random rows over a small alphabet of page ids (many accidental shared
    prefixes), random page size, GQA ratio and new-token counts."""
    rng = np.random.default_rng(seed)
    bs = int(rng.integers(2, 24))
    P = int(rng.choice([1, 2, 4, 16]))
    Hkv = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 4, 8]))
    width = int(rng.integers(1, 9))
    rows = rng.integers(0, int(rng.integers(1, 4)), size=(bs, width)).astype(np.int32)
    for j in range(1, bs):
        if rng.random() < 0.7:
            src = int(rng.integers(0, j))
            k = int(rng.integers(0, width + 1))
            rows[j, :k] = rows[src, :k]
    n = [int(x) for x in rng.choice([0, 1, 1, 1, 2, 5], size=bs)]
    L = [int(rng.integers(max(x, 1), width * P + 1)) if width * P >= max(x, 1) else max(x, 1)
         for x in n]
    W = max(-(-l // P) for l in L)
    if W > width:
        rows = np.concatenate([rows, np.zeros((bs, W - width), np.int32)], axis=1)
    return synth.build(f"rand{seed}", "bf16", G * Hkv, Hkv, 128, P, n, L, seed, rng, 1.0,
                       table=rows, num_pages=4)


@pytest.mark.parametrize("seed", range(30))
def test_detected_tree_matches_oracle_random(rp, seed):
    spec = random_shared_batch(seed)
    for mk in (1, 2 * spec.P, 5 * spec.P):
        p, got = plan_tree(rp, spec, prefix_detect_keys=mk)
        assert pt.canonical(got) == pt.canonical(oracle_tree(spec, mk)), (seed, mk)
        check_coverage(rp, p, spec)


def test_full_radix_tree_plans(rp):
    """The full-size radix workload (128 decodes, levels of 4096 / 8 x 2048 /
    4 x 1024 keys, shuffled order): detection finds the 1 + 8 + 32 levels, the
    partition's counts hold, and detection plus planning stays cheap."""
    spec = synth.radix_tree()
    p, got = plan_tree(rp, spec, prefix_detect_keys=256)
    sizes = sorted(len(nd["members"]) for nd in got)
    assert sizes == [4] * 32 + [16] * 8 + [128]
    assert sorted({nd["prefix"] for nd in got}) == [4096, 6144, 7168]
    info = p.info()
    assert info["cascade_depth"] == 3 and info["cascade_members"] == 128
    # each request's partials: its three levels' chunks plus its tail chunks
    times = []
    for _ in range(5):
        p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], spec.page_table)
        times.append(p.info()["plan_host_us"])
    assert min(times) < 5000, times


def test_cascade_tree_query_errors(rp):
    """The tree query reports CAPACITY when the arrays are too small, and the
    detection threshold must be >= 0."""
    import ctypes
    spec = synth.radix_tree_small(seed=43, shuffle=True)
    p, tree = plan_tree(rp, spec, prefix_detect_keys=1)
    inf = p.info()
    assert inf["num_cascade_levels"] == len(tree) == 7
    assert inf["num_cascade_level_members"] == sum(len(nd["members"]) for nd in tree)
    par = (ctypes.c_int32 * 8)()
    pre = (ctypes.c_int32 * 8)()
    ind = (ctypes.c_int32 * 9)()
    mem = (ctypes.c_int32 * 64)()
    st = rp.lib.rpkv_plan_get_cascade_tree(p._h, 6, 64, par, pre, ind, mem)
    assert st == 6  # CAPACITY: 7 levels do not fit 6
    st = rp.lib.rpkv_plan_get_cascade_tree(p._h, 8, inf["num_cascade_level_members"] - 1,
                                           par, pre, ind, mem)
    assert st == 6
    st = rp.lib.rpkv_plan_get_cascade_tree(p._h, 8, 64, par, pre, ind, mem)
    assert st == 0 and ind[7] == inf["num_cascade_level_members"]
    ok, _ = rp.supports(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=0,
                        max_batch=4, num_pages=64, max_tokens=64, max_pages_per_req=8,
                        prefix_detect_keys=-1)
    assert not ok


def test_detection_needs_the_host_table(rp):
    """Without a host copy of the page table there is nothing to detect from: the
    batch is planned without levels."""
    spec = synth.radix_tree_small(seed=44, shuffle=True)
    p = make_plan(rp, spec, prefix_detect_keys=1)
    p.plan_host(spec.cu_q, spec.L, spec.page_table.shape[1], None)
    assert p.cascade_tree() == [] and p.info()["cascade_members"] == 0
    check_coverage(rp, p, spec)
