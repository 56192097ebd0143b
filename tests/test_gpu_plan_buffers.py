"""GPU: the plan's fixed device buffers, the slot_mapping debug check, the
largest GQA ratios, and graph decode's length bound, through the C ABI against
the fp64 oracle (bars: store bit-exact, outputs within max-abs 2e-2 bf16)."""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_kv_store_amd as rp
from tests import gpu_harness as H
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def widen(spec, cols, num_pages):
    pt = np.zeros((spec.bs, cols), np.int32)
    pt[:, :spec.page_table.shape[1]] = spec.page_table
    return dataclasses.replace(spec, page_table=pt, num_pages=num_pages)


def test_prepare_allocates_once_small_then_maximal_batch():
    """One plan: a one-request batch, then a batch at every capacity (max_batch
    requests, max_tokens tokens, rows of max_pages_per_req pages), then small
    again.  The metadata capacity and the count of buffer allocations never
    change after the first prepare, and every batch matches the oracle."""
    B, Tm, W, P = 24, 700, 40, 16
    rng = np.random.default_rng(11)
    n_max = [300, 200] + [1] * 18 + [45] * 4          # 700 tokens
    L_max = [W * P, 250] + list(rng.integers(1, W * P + 1, 18)) + [W * P] * 4
    specs = [
        synth.build("one", "bf16", 32, 8, 128, P, [1], [77], 1, np.random.default_rng(1), 1.3),
        synth.build("max", "bf16", 32, 8, 128, P, n_max, L_max, 2, np.random.default_rng(2), 1.1),
        synth.build("mid", "bf16", 32, 8, 128, P, [60, 1, 1], [600, 333, 9], 3,
                    np.random.default_rng(3), 1.3),
    ]
    pages = max(s.num_pages for s in specs)
    specs = [widen(s, W, pages) for s in specs]
    plan = rp.Plan(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=P, dtype=rp.BF16,
                   max_batch=B, num_pages=pages, max_tokens=Tm, max_pages_per_req=W)
    caps, allocs = set(), set()
    for spec in specs:
        ht = synth.host_tensors(spec)
        ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
        db = H.dev_batch(spec, ht)
        out, _ = H.gpu_forward(spec, db, plan=plan)
        info = plan.info()
        assert info["metadata_bytes"] <= info["metadata_capacity_bytes"]
        caps.add(info["metadata_capacity_bytes"])
        allocs.add(info["buffer_allocations"])
        assert H.max_err(out, ref) <= 2e-2, spec.name
    assert len(caps) == 1 and allocs == {4}, (caps, allocs)


def test_check_slots_rejects_duplicates_before_any_write():
    spec = synth.small_config(2)
    ht = synth.host_tensors(spec)
    db = H.dev_batch(spec, ht)
    plan = H.make_plan(spec, check_slots=1)
    plan.prepare(spec.cu_q, spec.L, db.page_table, spec.page_table)
    k0, v0 = db.kpool.clone(), db.vpool.clone()
    bad = spec.slot_mapping.copy()
    bad[5] = bad[2]
    out = torch.full_like(db.q, 7.0)
    for call in ("store", "forward"):
        with pytest.raises(rp.RpkvError) as e:
            if call == "store":
                plan.store_kv(db.k, db.v, torch.from_numpy(bad).cuda(), db.kpool, db.vpool)
            else:
                plan.forward(db.q, db.k, db.v, torch.from_numpy(bad).cuda(), db.kpool, db.vpool,
                             out, spec.scale)
        assert e.value.status == 1 and "slot_mapping[5]" in str(e.value)
        torch.cuda.synchronize()
        assert torch.equal(db.kpool, k0) and torch.equal(db.vpool, v0)
        assert bool((out.float() == 7.0).all())
    oob = spec.slot_mapping.copy()
    oob[0] = spec.num_slots
    with pytest.raises(rp.RpkvError):
        plan.store_kv(db.k, db.v, torch.from_numpy(oob).cuda(), db.kpool, db.vpool)
    # valid slots pass the check and the step matches the oracle
    ref, _, kp_ref, _ = oracle.store_then_attend(spec, ht, nthreads=8)
    plan.forward(db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool, out, spec.scale)
    torch.cuda.synchronize()
    assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref)
    assert H.max_err(out, ref) <= 2e-2


GQA = [
    # name, Hq, Hkv, n, L: every request runs as MFMA tiles (n * G > 16), a
    # one-token tile holds G rows; a cascade hint is given and has no member
    ("g64", 64, 1, [150, 1, 1, 2, 40], [150, 700, 1300, 64, 300]),
    ("g64_hkv2", 128, 2, [33, 1, 1], [33, 900, 257]),
    ("g128", 128, 1, [70, 1, 1, 3], [70, 1100, 513, 90]),
]


@pytest.mark.parametrize("case", GQA, ids=[c[0] for c in GQA])
def test_largest_gqa_ratios_match_oracle(case):
    name, Hq, Hkv, n, L = case
    prefix = 64
    shared = ([1, 2], prefix)
    spec = synth.build(name, "bf16", Hq, Hkv, 128, 16, n, L, 8, np.random.default_rng(zlib.crc32(name.encode())),
                       1.3, shared=shared, groups=[(1, 2, prefix)])
    ht = synth.host_tensors(spec)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
    for tpb in (0, 1, 2):
        db = H.dev_batch(spec, ht)
        out, plan = H.gpu_forward(spec, db, tiles_per_block=tpb)
        info = plan.info()
        assert info["cascade_members"] == 0 and info["num_decode_items"] == 0
        assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref)
        assert np.array_equal(H.to_host_bits(spec, db.vpool), vp_ref)
        err = H.max_err(out, ref)
        assert err <= 2e-2, (name, tpb, err)


def test_graph_decode_skips_lengths_past_max_seq():
    """A request whose length exceeds the init's max_seq_len is skipped (its
    output rows are left as they were, no key is read past the page table's
    ceil(max_seq_len / P) columns); the others match the oracle."""
    from tests.test_gpu_graph_decode import graph_plan, uniform_batch
    bs, max_seq, P = 10, 1000, 16
    spec = uniform_batch("past_max", 32, 8, P, 1, bs, max_seq, np.random.default_rng(21))
    ht = synth.host_tensors(spec)
    ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    plan = graph_plan(spec, bs, 1, max_seq)
    lens = spec.L.copy()
    lens[3] = max_seq + 600          # out of range: skipped
    lens[7] = 0                      # below q_len: skipped
    out = torch.full_like(db.q, 5.0)
    cols = (max_seq + P - 1) // P    # exactly the columns the init requires
    pt = db.page_table[:, :cols].contiguous()
    plan.graph_decode_forward(bs, db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool,
                              torch.from_numpy(lens).cuda(), pt, out, spec.scale)
    torch.cuda.synchronize()
    got = H.to_f64(out)
    for i in range(bs):
        if i in (3, 7):
            assert np.all(got[i] == 5.0), i
        else:
            assert float(np.abs(got[i] - ref[i]).max()) <= 2e-2, i
