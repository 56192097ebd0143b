"""GPU: rpkv_graph_decode_forward_noalloc -- the graph-decode step with its
split-KV partials in the library's fixed device array, so no init and no
allocation -- against rpkv_graph_decode_forward (partials in buffers its init
allocated) on the same inputs: two calls in a row, the second with a smaller
batch; outputs within the bf16 bar of each other and of the fp64 oracle, pools
bit-exact.  A batch whose partials do not fit the array is refused with
RPKV_ERR_CAPACITY before anything is enqueued."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_kv_store_amd as rp
from tests import gpu_harness as H
from workloads import synth

pytestmark = pytest.mark.gpu

HQ, HKV, P = 32, 8, 16


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def uniform(name, bs, q_len, max_seq, seed):
    rng = np.random.default_rng(seed)
    L = rng.integers(q_len, max_seq + 1, bs).astype(np.int32)
    L[0], L[-1] = max_seq, q_len
    return synth.build(name, "bf16", HQ, HKV, 128, P, [q_len] * bs, L, seed, rng, 1.3)


def test_noalloc_matches_graph_decode_two_calls():
    calls = [("first", 48, 1, 3000, 61), ("second_smaller", 12, 2, 1500, 62)]
    specs = [uniform(*c[:2], c[2], c[3], c[4]) for c in calls]
    pages = max(s.num_pages for s in specs)
    cols = max(-(-c[3] // P) for c in calls)
    widened = []
    for s in specs:
        pt = np.zeros((s.bs, cols), np.int32)
        pt[:, :s.page_table.shape[1]] = s.page_table
        widened.append(dataclasses.replace(s, page_table=pt, num_pages=pages))
    plan = rp.Plan(num_q_heads=HQ, num_kv_heads=HKV, head_dim=128, page_size=P, dtype=rp.BF16,
                   max_batch=64, num_pages=pages, max_tokens=64, max_pages_per_req=cols)
    for (name, bs, q_len, max_seq, _), spec in zip(calls, widened):
        ht = synth.host_tensors(spec)
        ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
        lens = torch.from_numpy(spec.L).cuda()
        # the allocation-free entry point
        da = H.dev_batch(spec, ht)
        out_a = torch.full_like(da.q, float("nan"))
        plan.graph_decode_forward_noalloc(bs, q_len, max_seq, da.q, da.k, da.v, da.slot_mapping,
                                          da.kpool, da.vpool, lens, da.page_table, out_a,
                                          spec.scale)
        # the existing entry point on fresh copies of the same inputs
        db = H.dev_batch(spec, ht)
        gplan = rp.Plan(num_q_heads=HQ, num_kv_heads=HKV, head_dim=128, page_size=P,
                        dtype=rp.BF16, max_batch=bs, num_pages=pages, max_tokens=bs * q_len,
                        max_pages_per_req=cols)
        gplan.graph_decode_init(bs, q_len, max_seq)
        out_b = torch.full_like(db.q, float("nan"))
        gplan.graph_decode_forward(bs, db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool,
                                   lens, db.page_table, out_b, spec.scale)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out_a.float()).all()), name
        d = float((out_a.float() - out_b.float()).abs().max())
        print(f"{name}: noalloc vs graph decode max |diff| {d:.3e}, "
              f"bit-identical {torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))}")
        assert d <= 2e-2, name
        assert H.max_err(out_a, ref) <= 2e-2, name
        assert np.array_equal(H.to_host_bits(spec, da.kpool), kp_ref), name
        assert np.array_equal(H.to_host_bits(spec, da.vpool), vp_ref), name


def test_noalloc_refuses_partials_beyond_the_array():
    """1024 requests x 4 tokens over up to 8192 keys: two 4096-key chunks per
    request, 262144 partial rows of 129 floats, above 64 MiB.  Real buffers of
    the call's full size are passed (zero page ids, padding slots), yet nothing
    may be written."""
    bs, q_len, max_seq, pages = 1024, 4, 8192, 16
    cols = max_seq // P
    plan = rp.Plan(num_q_heads=HQ, num_kv_heads=HKV, head_dim=128, page_size=P, dtype=rp.BF16,
                   max_batch=bs, num_pages=pages, max_tokens=bs * q_len, max_pages_per_req=cols)
    T = bs * q_len
    q = torch.zeros((T, HQ, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((T, HKV, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    kp = torch.ones((pages * P, HKV, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.ones_like(kp)
    out = torch.full_like(q, 3.0)
    sm = torch.full((T,), -1, dtype=torch.int32, device="cuda")
    lens = torch.full((bs,), q_len, dtype=torch.int32, device="cuda")
    pt = torch.zeros((bs, cols), dtype=torch.int32, device="cuda")
    with pytest.raises(rp.RpkvError) as e:
        plan.graph_decode_forward_noalloc(bs, q_len, max_seq, q, k, v, sm, kp, vp, lens, pt, out,
                                          0.088)
    assert e.value.status == 6 and "no-alloc scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out.float() == 3.0).all()) and bool((kp.float() == 1.0).all())
