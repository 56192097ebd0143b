"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same
seeded inputs.  Bars: KV-pool store bit-exact; outputs within max-abs 2e-2
(bf16) / 1e-4 (fp32) of the oracle."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_kv_store_amd as rp
from tests import gpu_harness as H
from workloads import synth

pytestmark = pytest.mark.gpu


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _gpu():
    _require_gpu()
    yield


def check_full(spec, ht=None, groups=None, **plan_kw):
    ht = ht or synth.host_tensors(spec)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    out, plan = H.gpu_forward(spec, db, groups=groups, **plan_kw)
    assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref), "K pool differs after store"
    assert np.array_equal(H.to_host_bits(spec, db.vpool), vp_ref), "V pool differs after store"
    err = H.max_err(out, ref)
    assert err <= H.TOL[spec.dtype], f"{spec.name}: max abs err {err:.3e}"
    return err, plan, out, ref


# ---------------------------------------------------------------- small twins

@pytest.mark.parametrize("tpb", [0, 1, 2])
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_small_config_matches_oracle(cid, tpb):
    """tpb: MFMA tiles per workgroup (0: the planner's choice; 1: one tile per
    4-wavefront workgroup; 2: two tiles in ping-pong per 8-wavefront one)."""
    spec = synth.small_config(cid)
    err, plan, _, _ = check_full(spec, tiles_per_block=tpb)
    info = plan.info()
    if tpb and spec.dtype == "bf16" and info["num_prefill_items"]:
        assert info["tiles_per_block"] == tpb
    print(f"{spec.name}: max err {err:.2e} info {info}")


def test_cascade_equals_unsplit():
    spec = synth.small_config(5)
    ht = synth.host_tensors(spec)
    e1, p1, out1, ref = check_full(spec, ht)
    assert p1.info()["cascade_members"] == spec.groups[0][1]
    e2, p2, out2, _ = check_full(spec, ht, groups=[])
    assert p2.info()["cascade_members"] == 0
    assert float((out1.float() - out2.float()).abs().max()) <= 2e-2


@pytest.mark.parametrize("min_keys,target", [(32, 1 << 20), (64, 1 << 20), (256, 64),
                                             (2048, 0), (1 << 16, 0)])
def test_split_counts_match_oracle(min_keys, target):
    spec = synth.c3_decode_heavy(seed=21, scale=0.08, bs=12)
    err, plan, _, _ = check_full(spec, split_min_keys=min_keys, split_target=target)
    info = plan.info()
    print(info)


# ---------------------------------------------------------------- edge cases

EDGE = [
    # name, dtype, Hq, Hkv, P, n, L
    ("single_key", "bf16", 8, 8, 16, [1], [1]),
    ("n_equals_L_short", "bf16", 32, 8, 16, [5, 1], [5, 1]),
    ("zero_query_requests", "bf16", 32, 8, 16, [0, 3, 0, 1], [7, 40, 0, 90]),
    ("page1", "bf16", 16, 4, 1, [37, 1, 2], [37, 300, 70]),
    ("page4_ragged", "bf16", 16, 4, 4, [130, 1], [133, 77]),
    ("page64", "bf16", 16, 2, 64, [200, 1], [390, 1000]),
    ("page256", "bf16", 8, 1, 256, [3, 1], [700, 1500]),
    ("mha_g1", "bf16", 8, 8, 16, [150, 1, 1], [150, 513, 2]),
    ("g7_llama_like", "bf16", 28, 4, 16, [77, 1, 2], [301, 95, 64]),
    ("g16_decode_rows16", "bf16", 32, 2, 16, [1, 1], [333, 1025]),
    ("g32_prefill_path", "bf16", 32, 1, 16, [1, 3], [100, 67]),
    ("spec_decode_n2_g8", "bf16", 64, 8, 16, [2, 2, 3], [50, 513, 100]),
    ("threshold_n4_g4", "bf16", 32, 8, 16, [4, 5], [200, 200]),
    ("long_prefill_many_tiles", "bf16", 16, 2, 16, [700], [1500]),
    # the largest group sizes the bf16 kernels take: tiles of 2 tokens x 64
    # heads and of 1 token x 128 heads; decodes then run as tiles too
    ("g64_two_tokens_per_tile", "bf16", 64, 1, 16, [5, 1, 2], [300, 700, 41]),
    ("g128_one_token_per_tile", "bf16", 128, 1, 16, [3, 1, 1], [600, 257, 1]),
    ("g64_decodes_only", "bf16", 128, 2, 16, [1, 1, 1], [100, 2000, 5000]),
    ("f32_prefill_tiles", "f32", 8, 2, 4, [40, 1, 7], [40, 99, 30]),
    ("f32_page1_mha", "f32", 4, 4, 1, [9, 1], [20, 64]),
    # decode-only batches run the split-KV kernel on its own (K staged in LDS),
    # with per-key page lookups below 16 keys per page
    ("decode_only_page1", "bf16", 16, 4, 1, [1, 2, 1], [37, 300, 1000]),
    ("decode_only_page4", "bf16", 32, 8, 4, [1, 1, 3, 1], [5, 333, 777, 2050]),
    ("decode_only_page8", "bf16", 28, 4, 8, [2, 1], [2, 1500]),
    ("decode_only_page64", "bf16", 32, 2, 64, [1, 1, 1], [65, 129, 3000]),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_cases(case):
    name, dtype, Hq, Hkv, P, n, L = case
    D = 128
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    spec = synth.build(name, dtype, Hq, Hkv, D, P, n, L, 7, rng, 1.3)
    check_full(spec)


def test_empty_batch_is_a_no_op():
    spec = synth.build("empty", "bf16", 8, 2, 128, 16, [], [], 0, np.random.default_rng(0), 1.0)
    plan = H.make_plan(spec)
    pt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    plan.prepare(np.zeros(1, np.int32), np.zeros(0, np.int32), pt)
    q = torch.zeros((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    plan.attend(q, q, q, q, 0.1)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- probes

def test_poison_outside_rows_never_read():
    spec = synth.build("poison", "bf16", 32, 8, 128, 16, [300, 1, 2], [700, 900, 33], 3,
                       np.random.default_rng(3), 3.0)
    ht = synth.host_tensors(spec)
    ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
    used = np.zeros(spec.num_slots, bool)
    for i in range(spec.bs):
        used[synth.request_slots(spec.page_table[i], int(spec.L[i]), spec.P)] = True
    ht.kpool[~used] = synth.f32_to_bf16_bits(np.zeros(1, np.float32))[0]
    ht.vpool[~used] = synth.f32_to_bf16_bits(np.full(1, 8192.0, np.float32))[0]
    db = H.dev_batch(spec, ht)
    out, _ = H.gpu_forward(spec, db)
    assert H.max_err(out, ref) <= 2e-2


def _ramp(spec, ht, reverse=False):
    c = 256.0
    for i in range(spec.bs):
        slots = synth.request_slots(spec.page_table[i], int(spec.L[i]), spec.P)
        x = np.arange(int(spec.L[i]))
        K = np.zeros((len(x), spec.Hkv, spec.D), np.float32)
        K[:, :, 0] = (x >> 8)[:, None]
        K[:, :, 1] = (x & 255)[:, None]
        ht.kpool[slots] = synth.f32_to_bf16_bits(-K if reverse else K)
    q = np.zeros((spec.T, spec.Hq, spec.D), np.float32)
    q[:, :, 0] = 256 * c
    q[:, :, 1] = c
    ht.q[:] = synth.f32_to_bf16_bits(q)
    # the step's own keys must carry the ramp too: give k the ramp of its positions
    cu = spec.cu_q
    for i in range(spec.bs):
        pos = np.arange(int(spec.L[i]) - int(spec.n[i]), int(spec.L[i]))
        K = np.zeros((len(pos), spec.Hkv, spec.D), np.float32)
        K[:, :, 0] = (pos >> 8)[:, None]
        K[:, :, 1] = (pos & 255)[:, None]
        ht.k[cu[i]:cu[i + 1]] = synth.f32_to_bf16_bits(-K if reverse else K)


@pytest.mark.parametrize("n_new", [300, 270])
@pytest.mark.parametrize("tpb", [1, 2])
@pytest.mark.parametrize("reverse", [False, True])
def test_ramp_probe_pins_mask_boundary(reverse, tpb, n_new):
    """Each row's output is (within e^-20) the V row at its own position (or at
    position 0 for the reverse ramp): exercises the mask at every row, across
    tiles, splits, pages and both kernels.  The forward ramp's logits grow by
    thousands of base-2 units from step to step, so weights taken against the
    first step's max overflow: the paired tiles (tpb 2) must notice it and run
    again with the running max.  With 270 new tokens the chunk has 9 tiles, so
    one pair has a load-only partner group."""
    spec = synth.build("ramp", "bf16", 32, 8, 128, 16, [n_new, 1, 2, 1], [1000 + n_new, 2000, 513, 17], 5,
                       np.random.default_rng(5), 1.2)
    ht = synth.host_tensors(spec)
    _ramp(spec, ht, reverse)
    ref, _, kp, vp = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    out, plan = H.gpu_forward(spec, db, split_min_keys=64, tiles_per_block=tpb)
    assert plan.info()["tiles_per_block"] == tpb
    got = H.to_f64(out)
    cu = spec.cu_q
    for i in range(spec.bs):
        V = synth.as_float64(spec, vp[synth.request_slots(spec.page_table[i], int(spec.L[i]), spec.P)])
        for r in range(int(spec.n[i])):
            a = int(spec.L[i]) - int(spec.n[i]) + r
            want = V[0 if reverse else a]
            for h in range(spec.Hq):
                np.testing.assert_allclose(got[cu[i] + r, h], want[h // spec.G], atol=1e-2)
    assert H.max_err(out, ref) <= 2e-2


@pytest.mark.parametrize("tpb", [0, 2])
def test_needles_at_page_split_and_prefix_boundaries(tpb):
    """One dominant key placed around page, 32/64-key step, split-chunk and
    cascade-prefix boundaries: a row's output is that key's V iff it is visible.
    The needle's logit exceeds the others by about 65 base-2 units, so with two
    tiles per workgroup (tpb 2) a needle past a tile's first step takes the
    second, running-max pass in cascade-level and split tiles too."""
    prefix = 640
    n_share = 6
    tails = [70, 100, 130, 64, 65, 200]
    L = [prefix + t for t in tails] + [900]
    n = [1] * n_share + [200]
    spec = synth.build("needle", "bf16", 32, 8, 128, 16, n, L, 9, np.random.default_rng(9), 1.2,
                       shared=(list(range(n_share)), prefix), groups=[(0, n_share, prefix)])
    base = synth.host_tensors(spec)
    for p in (15, 16, 63, 64, 255, 256, 639, 640, 641, 767, 768, 899):
        ht = synth.HostTensors(base.kpool.copy(), base.vpool.copy(), base.q.copy(),
                               base.k.copy(), base.v.copy())
        q = np.zeros((spec.T, spec.Hq, spec.D), np.float32)
        q[:, :, 5] = 8.0
        ht.q[:] = synth.f32_to_bf16_bits(q)
        Kn = np.zeros((spec.Hkv, spec.D), np.float32)
        Kn[:, 5] = 64.0  # logit 8*64/sqrt(128) = 45 against ~0 elsewhere
        cu = spec.cu_q
        for i in range(spec.bs):
            if p >= int(spec.L[i]):
                continue
            s = synth.request_slots(spec.page_table[i], int(spec.L[i]), spec.P)[p]
            t_new = p - (int(spec.L[i]) - int(spec.n[i]))
            if t_new >= 0:
                ht.k[cu[i] + t_new] = synth.f32_to_bf16_bits(Kn)
            else:
                ht.kpool[s] = synth.f32_to_bf16_bits(Kn)
        # keep every other key's logit at 0: zero q components elsewhere already
        ref, _, kp, vp = oracle.store_then_attend(spec, ht, nthreads=8)
        db = H.dev_batch(spec, ht)
        out, plan = H.gpu_forward(spec, db, split_min_keys=64, tiles_per_block=tpb)
        assert plan.info()["cascade_members"] == n_share
        assert H.max_err(out, ref) <= 2e-2, p


# ---------------------------------------------------------------- invariants

def test_mixed_pass_equals_each_request_alone():
    spec = synth.small_config(2)
    ht = synth.host_tensors(spec)
    err, plan, out_mixed, ref = check_full(spec, ht)
    cu = spec.cu_q
    for i in range(spec.bs):
        sub = synth.BatchSpec(spec.name, spec.dtype, spec.Hq, spec.Hkv, spec.D, spec.P,
                              spec.num_pages, spec.n[i:i + 1].copy(), spec.L[i:i + 1].copy(),
                              spec.page_table[i:i + 1].copy(), spec.slot_mapping[cu[i]:cu[i + 1]],
                              [], spec.seed)
        sht = synth.HostTensors(ht.kpool, ht.vpool, ht.q[cu[i]:cu[i + 1]], ht.k[cu[i]:cu[i + 1]],
                                ht.v[cu[i]:cu[i + 1]])
        db = H.dev_batch(sub, sht)
        out, _ = H.gpu_forward(sub, db)
        d = float((out.float() - out_mixed[cu[i]:cu[i + 1]].float()).abs().max())
        assert d <= 2e-2, (i, d)


def test_decode_equals_last_row_of_full_prefill():
    L = 777
    spec = synth.build("full", "bf16", 32, 8, 128, 16, [L], [L], 4, np.random.default_rng(4), 1.0)
    ht = synth.host_tensors(spec)
    _, _, out_full, ref = check_full(spec, ht)
    dec = synth.BatchSpec("dec", "bf16", 32, 8, 128, 16, spec.num_pages, np.array([1], np.int32),
                          np.array([L], np.int32), spec.page_table, spec.slot_mapping[L - 1:],
                          [], 4)
    dht = synth.HostTensors(ht.kpool, ht.vpool, ht.q[L - 1:], ht.k[L - 1:], ht.v[L - 1:])
    # the decode step sees the earlier tokens' K/V already stored
    kp, vp = ht.kpool.copy(), ht.vpool.copy()
    oracle.store_kv(kp, vp, ht.k, ht.v, spec.slot_mapping)
    dht = synth.HostTensors(kp, vp, ht.q[L - 1:], ht.k[L - 1:], ht.v[L - 1:])
    db = H.dev_batch(dec, dht)
    out, plan = H.gpu_forward(dec, db, split_min_keys=64)
    assert plan.info()["num_decode_items"] > 1
    assert float((out[0].float() - out_full[L - 1].float()).abs().max()) <= 2e-2
    assert H.max_err(out, ref[L - 1:]) <= 2e-2


def test_store_kv_bitwise_with_padding_slots():
    spec = synth.small_config(4)
    ht = synth.host_tensors(spec)
    db = H.dev_batch(spec, ht)
    sm = spec.slot_mapping.copy()
    sm[::7] = -1                       # padding tokens
    sm[3] = spec.num_slots + 5         # out of range: skipped, never written
    plan = H.make_plan(spec)
    plan.store_kv(db.k, db.v, torch.from_numpy(sm).cuda(), db.kpool, db.vpool)
    torch.cuda.synchronize()
    kp, vp = ht.kpool.copy(), ht.vpool.copy()
    keep = (sm >= 0) & (sm < spec.num_slots)
    kp[sm[keep]] = ht.k[keep]
    vp[sm[keep]] = ht.v[keep]
    assert np.array_equal(H.to_host_bits(spec, db.kpool), kp)
    assert np.array_equal(H.to_host_bits(spec, db.vpool), vp)


def test_one_prepare_serves_many_layers_and_plans_are_reusable():
    """One prepare serves several layers (different pools and q/k/v); one plan
    then serves batches of different sizes (its device buffers grow and shrink).
    Every batch has the plan's head shape and pool size."""
    import dataclasses
    big = synth.c2_llama8b_mixed(seed=31, scale=0.2)
    small = synth.c2_llama8b_mixed(seed=32, scale=0.1)
    pool_pages = max(big.num_pages, small.num_pages)
    cols = max(big.page_table.shape[1], small.page_table.shape[1])

    def widen(spec):
        pt = np.zeros((spec.bs, cols), np.int32)
        pt[:, :spec.page_table.shape[1]] = spec.page_table
        return dataclasses.replace(spec, num_pages=pool_pages, page_table=pt)

    big, small = widen(big), widen(small)
    plan = rp.Plan(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype=rp.BF16,
                   max_batch=8, num_pages=pool_pages, max_tokens=max(big.T, small.T),
                   max_pages_per_req=cols)
    for layer in range(3):
        ht = synth.host_tensors(small, seed=100 + layer)
        ref, _, _, _ = oracle.store_then_attend(small, ht, nthreads=8)
        db = H.dev_batch(small, ht)
        if layer == 0:
            plan.prepare(small.cu_q, small.L, db.page_table, small.page_table)
        out = torch.empty_like(db.q)
        plan.forward(db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool, out, small.scale)
        torch.cuda.synchronize()
        assert H.max_err(out, ref) <= 2e-2
    for spec in (big, small):
        ht = synth.host_tensors(spec)
        ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
        db = H.dev_batch(spec, ht)
        out, _ = H.gpu_forward(spec, db, plan=plan)
        assert H.max_err(out, ref) <= 2e-2


def test_binding_rejects_tensors_of_another_shape():
    spec = synth.small_config(2)
    ht = synth.host_tensors(spec)
    db = H.dev_batch(spec, ht)
    plan = H.make_plan(spec)
    plan.prepare(spec.cu_q, spec.L, db.page_table, spec.page_table)
    out = torch.empty_like(db.q)
    with pytest.raises(ValueError):
        plan.forward(db.q[:, :16].contiguous(), db.k, db.v, db.slot_mapping, db.kpool, db.vpool,
                     out, spec.scale)
    with pytest.raises(ValueError):
        plan.forward(db.q, db.k, db.v, db.slot_mapping, db.kpool[:-16].contiguous(), db.vpool,
                     out, spec.scale)
    with pytest.raises(ValueError):
        plan.forward(db.q.float(), db.k, db.v, db.slot_mapping, db.kpool, db.vpool, out,
                     spec.scale)


@pytest.mark.parametrize("P", [16, 4, 1])
def test_tile_pairs_of_unequal_lengths(P):
    """Tiles in ping-pong pairs whose step counts differ (1 to 14 steps, ranges
    ending mid-step, an odd number of tiles so one pair has an empty partner)
    equal the oracle, and equal the same batch run one tile per workgroup."""
    n = [1, 37, 64, 65, 130, 40, 200]
    L = [1, 37 + 300, 64, 65 + 700, 130 + 64, 40 + 5, 200 + 651]
    spec = synth.build(f"pairs_p{P}", "bf16", 8, 2, 128, P, n, L, 77, np.random.default_rng(77), 1.2)
    ht = synth.host_tensors(spec)
    e2, p2, out2, _ = check_full(spec, ht, tiles_per_block=2)
    e1, p1, out1, _ = check_full(spec, ht, tiles_per_block=1)
    assert p2.info()["tiles_per_block"] == 2 and p1.info()["tiles_per_block"] == 1
    assert float((out1.float() - out2.float()).abs().max()) <= 2e-2
    print(f"{spec.name}: err pairs {e2:.2e} single {e1:.2e}")


# ---------------------------------------------------------------- full size

@pytest.mark.parametrize("cid,tpb", [(1, 0), (2, 0), (3, 0), (4, 0), (5, 0), (2, 2), (4, 1), (5, 1)])
def test_full_size_sampled_rows(cid, tpb):
    """The five workloads at their stated sizes, in the launch configuration the
    benchmark times (tpb 0: the planner picks the tiles per workgroup, as in the
    benchmark), plus the other tile arrangement for the prefill-heavy ones;
    sampled requests and rows are checked against the oracle on the sub-problem
    of exactly the pages they reference; the store is checked bit-exact on those
    pages."""
    spec = synth.full_config(cid)
    rng = np.random.default_rng(cid)
    if cid == 1:
        ht = synth.host_tensors(spec)
        check_full(spec, ht)
        return
    db = H.device_contents(spec, seed=1000 + cid)
    reqs = H.pick_requests(spec, rng)
    sub = H.subproblem(spec, db, reqs)          # taken before the store
    rows = H.pick_rows(spec, reqs, rng)
    sub_rows = rows[sub.token_map]
    out, plan = H.gpu_forward(spec, db, tiles_per_block=tpb)
    if tpb:
        assert plan.info()["tiles_per_block"] == tpb
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(sub.spec, sub.tensors, rows=sub_rows,
                                                      nthreads=8)
    got = H.to_f64(out[torch.from_numpy(sub.token_map).cuda()])
    err = float(np.abs(got[sub_rows] - ref[sub_rows]).max())
    print(f"{spec.name}: {int(sub_rows.sum())} rows of {len(reqs)} requests, max err {err:.2e}")
    assert err <= H.TOL[spec.dtype]
    P = spec.P
    pg = torch.from_numpy(sub.pages).cuda()
    kp_gpu = db.kpool.view(spec.num_pages, P, spec.Hkv, spec.D)[pg].reshape(-1, spec.Hkv, spec.D)
    vp_gpu = db.vpool.view(spec.num_pages, P, spec.Hkv, spec.D)[pg].reshape(-1, spec.Hkv, spec.D)
    assert np.array_equal(H.to_host_bits(spec, kp_gpu), kp_ref)
    assert np.array_equal(H.to_host_bits(spec, vp_gpu), vp_ref)
    # every output row is finite
    assert bool(torch.isfinite(out.float()).all())
