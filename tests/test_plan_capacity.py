"""Host-side tests (no GPU) of the plan's fixed metadata capacity and of the
slot_mapping check.

A plan sizes its device metadata buffer once, from the shape's capacities
(max_batch, max_tokens, max_pages_per_req), so prepare never allocates.  These
tests plan batches built to push each term of that bound -- many short prefill
tiles, key-split tiles, deep nested cascade levels, many split-KV chunks, very
unequal tile lengths for the XCD queues, fp32 one-token tiles -- and check that
every batch's partition fits the capacity, that the capacity never changes, and
that the partitions still cover every visible (token, head, key) exactly once."""
import numpy as np
import pytest

from tests.test_abi_host import check_coverage
from workloads import synth


@pytest.fixture(scope="module")
def rp():
    import ragged_paged_kv_store_amd as rp
    return rp


def plan_for(rp, Hq, Hkv, P, max_batch, max_tokens, max_pages, dtype=0, **kw):
    return rp.Plan(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=P, dtype=dtype,
                   max_batch=max_batch, num_pages=1 << 20, max_tokens=max_tokens,
                   max_pages_per_req=max_pages, **kw)


def plan_and_check(rp, plan, spec, groups=None, coverage=True):
    cols = plan.shape.max_pages_per_req
    pt = np.zeros((spec.bs, cols), np.int32)
    pt[:, :spec.page_table.shape[1]] = spec.page_table
    plan.plan_host(spec.cu_q, spec.L, cols, pt, spec.groups if groups is None else groups)
    info = plan.info()
    assert 0 < info["metadata_bytes"] <= info["metadata_capacity_bytes"], info
    if coverage:
        check_coverage(rp, plan, spec)
    return info


def spec_of(name, Hq, Hkv, P, n, L, seed=0, dtype="bf16", shared=None, groups=None):
    return synth.build(name, dtype, Hq, Hkv, 128, P, n, L, seed, np.random.default_rng(seed),
                       1.0, shared=shared, groups=groups)


def test_capacity_is_fixed_and_holds_extreme_batches(rp):
    """One plan, many batches at its limits: the capacity it reports never
    changes and every batch fits it."""
    B, Tm, W, P = 64, 4096, 512, 16
    plan = plan_for(rp, 32, 8, P, B, Tm, W, split_min_keys=32, split_target=1 << 20)
    cap = None
    rng = np.random.default_rng(1)
    batches = [
        # many 5-token prefill-type requests (n * G > 16): one short tile each
        ([5] * B, [5 + 7 * i for i in range(B)]),
        # every token in one long prefill: key splits of the long tiles
        ([Tm], [W * P]),
        # decodes at the longest row: the most split-KV chunks
        ([1] * B, [W * P] * B),
        # one long request and many one-step tiles (very unequal XCD queues)
        ([2000] + [5] * (B - 1), [W * P] + [5] * (B - 1)),
        # random mixes
        *[(list(n), [int(rng.integers(max(x, 1), W * P + 1)) for x in n])
          for n in (rng.integers(0, 60, size=B) for _ in range(6))],
    ]
    for k, (n, L) in enumerate(batches):
        spec = spec_of(f"cap{k}", 32, 8, P, n, L, seed=k)
        info = plan_and_check(rp, plan, spec, coverage=k != 1)
        cap = cap or info["metadata_capacity_bytes"]
        assert info["metadata_capacity_bytes"] == cap


@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_deep_nested_cascade_fits_and_is_capped(rp, G):
    """Nested hints 20 levels deep: the planner keeps the top 16 levels, the rest
    of the keys go to the members' tails; the partition is exactly-once and fits
    the capacity."""
    P, depth = 4, 20
    B = depth + 2
    n = [max(1, 16 // G // 2)] * B
    L = [P * (depth + 3) + i for i in range(B)]
    # level k holds requests 0 .. B-1-k, sharing k+1 pages: request r >= 1
    # shares its first min(depth, B - r) pages with request 0
    spec = spec_of(f"deep{G}", 2 * G, 2, P, n, L, seed=G)
    pt = spec.page_table.copy()
    for r in range(1, B):
        s = min(depth, B - r)
        pt[r, :s] = pt[0, :s]
    groups = [(0, B - k, P * (k + 1)) for k in range(depth)]
    spec = synth.build(spec.name, "bf16", 2 * G, 2, 128, P, n, L, 0, np.random.default_rng(0), 1.0,
                       table=pt, num_pages=spec.num_pages, groups=groups)
    plan = plan_for(rp, 2 * G, 2, P, B, sum(n), depth + 12)
    info = plan_and_check(rp, plan, spec)
    assert info["cascade_depth"] == 16
    assert info["num_cascade_levels"] == 16
    # detection finds the same chain and is capped the same way
    plan2 = plan_for(rp, 2 * G, 2, P, B, sum(n), depth + 12, prefix_detect_keys=1)
    info2 = plan_and_check(rp, plan2, spec, groups=[])
    assert info2["cascade_depth"] == 16


def test_fp32_one_token_tiles_fit(rp):
    """fp32 at G = 16: one token per 16-row tile, the most items per token."""
    n = [40, 1, 7, 300]
    L = [40, 99, 30, 600]
    spec = spec_of("f32g16", 16, 1, 4, n, L, dtype="f32")
    plan = plan_for(rp, 16, 1, 4, 4, sum(n), 160, dtype=1)
    plan_and_check(rp, plan, spec)


def test_check_slot_mapping(rp):
    plan = plan_for(rp, 32, 8, 16, 4, 64, 8)
    num_slots = (1 << 20) * 16
    plan.check_slot_mapping([5, -1, 9, -1, 7])          # padding (-1) may repeat
    plan.check_slot_mapping([])
    with pytest.raises(rp.RpkvError) as e:
        plan.check_slot_mapping([5, 6, 9, 6, 7])
    assert e.value.status == 1 and "slot_mapping[3]" in str(e.value) and "token 1" in str(e.value)
    with pytest.raises(rp.RpkvError) as e:
        plan.check_slot_mapping([5, num_slots, 9])
    assert e.value.status == 1 and "slot_mapping[1]" in str(e.value)
    # the first duplicate reported is the earliest repeating token
    with pytest.raises(rp.RpkvError) as e:
        plan.check_slot_mapping([1, 2, 3, 3, 1])
    assert "slot_mapping[3]" in str(e.value)
    # a real batch's slots are distinct
    spec = synth.full_config(4)
    big = rp.Plan(num_q_heads=spec.Hq, num_kv_heads=spec.Hkv, head_dim=128, page_size=spec.P,
                  dtype=0, max_batch=spec.bs, num_pages=spec.num_pages, max_tokens=spec.T,
                  max_pages_per_req=spec.page_table.shape[1])
    big.check_slot_mapping(spec.slot_mapping)
    dup = spec.slot_mapping.copy()
    dup[-1] = dup[0]
    with pytest.raises(rp.RpkvError):
        big.check_slot_mapping(dup)
