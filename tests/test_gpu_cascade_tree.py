"""GPU parity of the multi-level cascade: shared-prefix levels found from the page
table (or given as nested hints) are attended once per level, stacked in MFMA
tiles, and merged with each request's tail by log-sum-exp.  The result must equal
plain attention -- the fp64 oracle on the same seeded inputs -- within 2e-2
(bf16), with the KV-pool store bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from oracle import prefix_tree as pt
from tests import gpu_harness as H
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def decode_type(spec):
    return [bool(n > 0 and n * spec.G <= 16) for n in spec.n]


def check(spec, groups=(), ht=None, **plan_kw):
    ht = ht or synth.host_tensors(spec)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    out, plan = H.gpu_forward(spec, db, groups=list(groups), **plan_kw)
    assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref), "K pool differs after store"
    assert np.array_equal(H.to_host_bits(spec, db.vpool), vp_ref), "V pool differs after store"
    err = H.max_err(out, ref)
    print(f"{spec.name} P={spec.P}: max err {err:.2e} info {plan.info()}")
    assert err <= H.TOL[spec.dtype], f"{spec.name}: max abs err {err:.3e}"
    return plan, out


@pytest.mark.parametrize("P", [1, 4, 16, 64])
def test_detected_levels_match_oracle(P):
    spec = synth.radix_tree_small(seed=50 + P, shuffle=True, P=P)
    plan, _ = check(spec, prefix_detect_keys=1)
    info = plan.info()
    assert info["cascade_depth"] == 3 and info["cascade_members"] == 16
    tree = plan.cascade_tree()
    assert pt.canonical(tree) == pt.canonical(
        pt.prefix_tree(spec.page_table, spec.L, spec.n, spec.P, decode_type(spec), 1))


def test_nested_hints_match_oracle():
    spec = synth.radix_tree_small(seed=61, shuffle=False)
    plan, _ = check(spec, groups=spec.groups)
    assert plan.info()["cascade_depth"] == 3


def test_levels_not_aligned_to_key_tiles():
    """Level boundaries at 80, 128 and 144 keys: level tiles and tails start
    inside a 64-key tile and inside a 32-key decode step."""
    spec = synth.radix_tree_small(seed=62, shuffle=True, levels=((1, 80), (2, 48), (2, 16)))
    plan, _ = check(spec, prefix_detect_keys=1)
    assert plan.info()["cascade_depth"] == 3


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 8), (8, 8), (28, 4)])
def test_gqa_ratios(Hq, Hkv):
    spec = synth.radix_tree_small(seed=63 + Hq, shuffle=True, Hq=Hq, Hkv=Hkv)
    plan, _ = check(spec, prefix_detect_keys=1)
    assert plan.info()["cascade_members"] == 16


def test_mixed_batch_with_prefills():
    """Levels beside prefill-type requests in one fused launch."""
    spec = synth.radix_tree_small(seed=64, shuffle=True, extra_prefills=((300, 80), (0, 64)))
    plan, _ = check(spec, prefix_detect_keys=1)
    assert plan.info()["cascade_depth"] == 3


def test_pruned_levels_and_cascade_off_agree():
    spec = synth.radix_tree_small(seed=65, shuffle=True)
    ht = synth.host_tensors(spec)
    outs = []
    for mk in (1, 150, 0):
        plan, out = check(spec, ht=ht, prefix_detect_keys=mk)
        outs.append(out.float())
        if mk == 150:
            assert plan.info()["cascade_depth"] == 2   # the 128-key level folds into the 64-key one
        if mk == 0:
            assert plan.info()["cascade_members"] == 0
    assert float((outs[0] - outs[2]).abs().max()) <= 2e-2
    assert float((outs[1] - outs[2]).abs().max()) <= 2e-2


def test_repeated_prepare_reuses_plan():
    """One plan across batches with different trees (deeper, then one level,
    then two) gives the oracle's result each time."""
    specs = [synth.radix_tree_small(seed=seed, shuffle=True, levels=levels)
             for seed, levels in ((66, None), (67, ((1, 64),)), (68, ((2, 128), (2, 64))))]
    s0 = specs[0]
    maxp = max(s.num_pages for s in specs)
    for s in specs:
        s.num_pages = maxp   # one pool size for the plan; unused pages stay random
    plan = H.rp.Plan(num_q_heads=s0.Hq, num_kv_heads=s0.Hkv, head_dim=s0.D, page_size=s0.P,
                     dtype=H.rp.BF16, max_batch=max(s.bs for s in specs),
                     num_pages=maxp,
                     max_tokens=max(s.T for s in specs),
                     max_pages_per_req=max(s.page_table.shape[1] for s in specs),
                     prefix_detect_keys=1)
    for spec, depth in zip(specs, (3, 1, 2)):
        ht = synth.host_tensors(spec)
        ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
        db = H.dev_batch(spec, ht)
        out, _ = H.gpu_forward(spec, db, groups=[], plan=plan)
        assert plan.info()["cascade_depth"] == depth
        assert H.max_err(out, ref) <= 2e-2


def test_full_size_radix_tree_sampled_rows():
    """The full radix workload (128 decodes, levels 4096 / 8 x 2048 / 4 x 1024
    keys, shuffled order, level threshold 256 keys) in the benchmark's launch
    configuration; sampled requests are checked against the oracle on the
    sub-problem of the pages they reference, and the store bit-exact there."""
    spec = synth.radix_tree()
    rng = np.random.default_rng(7)
    db = H.device_contents(spec, seed=1006)
    reqs = H.pick_requests(spec, rng, max_reqs=12)
    sub = H.subproblem(spec, db, reqs)
    rows = H.pick_rows(spec, reqs, rng)
    sub_rows = rows[sub.token_map]
    out, plan = H.gpu_forward(spec, db, groups=[], prefix_detect_keys=256)
    info = plan.info()
    assert info["cascade_depth"] == 3 and info["num_cascade_levels"] == 41
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(sub.spec, sub.tensors, rows=sub_rows,
                                                      nthreads=8)
    got = H.to_f64(out[torch.from_numpy(sub.token_map).cuda()])
    err = float(np.abs(got[sub_rows] - ref[sub_rows]).max())
    print(f"{spec.name}: {int(sub_rows.sum())} rows of {len(reqs)} requests, max err {err:.2e}")
    assert err <= 2e-2
    P = spec.P
    pg = torch.from_numpy(sub.pages).cuda()
    kp_gpu = db.kpool.view(spec.num_pages, P, spec.Hkv, spec.D)[pg].reshape(-1, spec.Hkv, spec.D)
    vp_gpu = db.vpool.view(spec.num_pages, P, spec.Hkv, spec.D)[pg].reshape(-1, spec.Hkv, spec.D)
    assert np.array_equal(H.to_host_bits(spec, kp_gpu), kp_ref)
    assert np.array_equal(H.to_host_bits(spec, vp_gpu), vp_ref)
    assert bool(torch.isfinite(out.float()).all())


@pytest.mark.parametrize("D", [64, 128])
def test_f32_levels(D):
    """fp32 batches: the levels run on the fp32 tiles (16 rows) and split-KV path."""
    spec = synth.radix_tree_small(seed=70 + D, shuffle=True, dtype="f32", D=D)
    plan, _ = check(spec, prefix_detect_keys=1)
    assert plan.info()["cascade_depth"] == 3


def test_csr_page_table_detects_the_same_levels():
    """With the page table in CSR form (and its host copy) the planner finds the
    same levels and the outputs are bit-identical to the dense table's."""
    from tests.test_gpu_page_formats import bits, to_csr
    spec = synth.radix_tree_small(seed=72, shuffle=True)
    ht = synth.host_tensors(spec)
    out_dense, p1 = H.gpu_forward(spec, H.dev_batch(spec, ht), groups=[], prefix_detect_keys=1)
    db = H.dev_batch(spec, ht)
    indptr, indices, last = to_csr(spec)
    plan = H.make_plan(spec, prefix_detect_keys=1)
    plan.prepare_csr(spec.cu_q, indptr, last, torch.from_numpy(indices).cuda(), indices)
    out = torch.full_like(db.q, float("nan"))
    plan.forward(db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool, out, spec.scale)
    torch.cuda.synchronize()
    assert pt.canonical(plan.cascade_tree()) == pt.canonical(p1.cascade_tree())
    assert plan.info()["cascade_depth"] == 3
    assert torch.equal(bits(out), bits(out_dense))
