"""GPU: the graph-capturable decode path (rpkv_graph_decode_init/forward) on
uniform decode batches: eager calls against the fp64 oracle (outputs within the
bf16 bar, pools bit-exact), and one captured HIP graph replayed with new
lengths, slots and contents written in place, every replay against the oracle."""
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


def uniform_batch(name, Hq, Hkv, P, q_len, bs, max_seq, rng):
    L = rng.integers(q_len, max_seq + 1, bs).astype(np.int32)
    # lengths at the edges: q_len itself, chunk-ish multiples and the maximum
    for j, x in enumerate([q_len, max_seq, 256, 257, 1024, 1023]):
        if j < bs and q_len <= x <= max_seq:
            L[j] = x
    cols = (max_seq + P - 1) // P
    spec = synth.build(name, "bf16", Hq, Hkv, 128, P, [q_len] * bs, L, 5, rng, 1.3)
    pt = np.zeros((bs, cols + 2), np.int32)
    pt[:, :spec.page_table.shape[1]] = spec.page_table
    return dataclasses.replace(spec, page_table=pt)


def graph_plan(spec, max_batch, q_len, max_seq):
    plan = rp.Plan(num_q_heads=spec.Hq, num_kv_heads=spec.Hkv, head_dim=128, page_size=spec.P,
                   dtype=rp.BF16, max_batch=max_batch, num_pages=spec.num_pages,
                   max_tokens=max_batch * q_len, max_pages_per_req=spec.page_table.shape[1])
    plan.graph_decode_init(max_batch, q_len, max_seq)
    return plan


CASES = [
    # name, Hq, Hkv, P, q_len, bs, max_seq
    ("g4_q1", 32, 8, 16, 1, 64, 4096),
    ("g8_q2", 64, 8, 16, 2, 17, 3000),
    ("g4_page1", 16, 4, 1, 1, 9, 600),
    ("g16_q1_long", 32, 2, 64, 1, 5, 9000),
    ("g7_q2", 28, 4, 16, 2, 33, 2048),
    ("short_single_chunk", 32, 8, 16, 1, 12, 200),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_decode_matches_oracle(case):
    name, Hq, Hkv, P, q_len, bs, max_seq = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    spec = uniform_batch(name, Hq, Hkv, P, q_len, bs, max_seq, rng)
    ht = synth.host_tensors(spec)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    plan = graph_plan(spec, bs + 3, q_len, max_seq)
    out = torch.full_like(db.q, float("nan"))
    lens = torch.from_numpy(spec.L).cuda()
    plan.graph_decode_forward(bs, db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool, lens,
                              db.page_table, out, spec.scale)
    torch.cuda.synchronize()
    assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref)
    assert np.array_equal(H.to_host_bits(spec, db.vpool), vp_ref)
    err = H.max_err(out, ref)
    assert err <= H.TOL["bf16"], f"{name}: max abs err {err:.3e}"


def random_graph_case(seed):
    rng = np.random.default_rng(7000 + seed)
    G = int(rng.choice([1, 2, 4, 7, 8, 16]))
    q_len = int(rng.integers(1, min(16 // G, 3) + 1))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.choice([1, 4, 16, 64]))
    bs = int(rng.integers(1, 41))
    max_seq = int(rng.integers(q_len, 8001))
    return (f"random{seed}", G * Hkv, Hkv, P, q_len, bs, max_seq)


@pytest.mark.parametrize("seed", range(32))
def test_graph_decode_random_shapes(seed):
    """Seeded uniform batches of random GQA ratio, KV heads, page size, q_len,
    batch and max_seq_len, eager calls against the oracle."""
    test_graph_decode_matches_oracle(random_graph_case(seed))


def test_graph_decode_equals_planned_path():
    spec = uniform_batch("eq", 32, 8, 16, 1, 40, 5000, np.random.default_rng(5))
    ht = synth.host_tensors(spec)
    db = H.dev_batch(spec, ht)
    k0, v0 = db.kpool.clone(), db.vpool.clone()
    out1, _ = H.gpu_forward(spec, db)
    db.kpool.copy_(k0)
    db.vpool.copy_(v0)
    plan = graph_plan(spec, 40, 1, 5000)
    out2 = torch.full_like(db.q, float("nan"))
    plan.graph_decode_forward(40, db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool,
                              torch.from_numpy(spec.L).cuda(), db.page_table, out2, spec.scale)
    torch.cuda.synchronize()
    assert float((out1.float() - out2.float()).abs().max()) <= 2e-2


def test_graph_capture_replays_with_new_lengths():
    """One capture, five replays; before each, new lengths, slots (built on the
    device from the lengths and the page table), q/k/v are written in place."""
    bs, q_len, max_seq, Hq, Hkv, P = 16, 1, 2000, 32, 8, 16
    rng = np.random.default_rng(7)
    base = uniform_batch("replay", Hq, Hkv, P, q_len, bs, max_seq, rng)
    base = dataclasses.replace(base, L=np.full(bs, max_seq, np.int32))
    # every row's pages cover max_seq: allocate a fresh table over the pool
    cols = base.page_table.shape[1]
    need = (max_seq + P - 1) // P
    num_pages = max(base.num_pages, need * bs)
    pages = rng.permutation(num_pages)[:need * bs].reshape(bs, need).astype(np.int32)
    pt = np.zeros((bs, cols), np.int32)
    pt[:, :need] = pages
    spec0 = dataclasses.replace(base, page_table=pt, num_pages=num_pages)
    ht0 = synth.host_tensors(spec0)
    kp_host, vp_host = ht0.kpool, ht0.vpool
    kpool, vpool = H.to_dev(spec0, kp_host), H.to_dev(spec0, vp_host)
    pt_d = torch.from_numpy(pt).cuda()
    lens_d = torch.full((bs,), max_seq, dtype=torch.int32, device="cuda")
    nc_d = torch.zeros(bs, dtype=torch.int32, device="cuda")
    n_d = torch.full((bs,), q_len, dtype=torch.int32, device="cuda")
    T = bs * q_len
    q_d = torch.zeros((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    k_d = torch.zeros((T, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    v_d = torch.zeros_like(k_d)
    out_d = torch.zeros_like(q_d)
    meta = {k: torch.empty(sz, dtype=torch.int32, device="cuda") for k, sz in
            (("query_start_loc", bs + 1), ("seq_lens", bs), ("positions", T),
             ("slot_mapping", T), ("logits_indices", bs), ("counts", 2))}
    plan = graph_plan(spec0, bs, q_len, max_seq)

    def step(stream):
        rp.build_metadata(nc_d, n_d, pt_d, P, max_tokens=T, out=meta, stream=stream)
        plan.graph_decode_forward(bs, q_d, k_d, v_d, meta["slot_mapping"], kpool, vpool,
                                  meta["seq_lens"], pt_d, out_d, spec0.scale, stream=stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(s.cuda_stream)  # warm-up outside capture
    torch.cuda.synchronize()
    kpool.copy_(H.to_dev(spec0, kp_host))
    vpool.copy_(H.to_dev(spec0, vp_host))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(5):
        L = rng.integers(q_len, max_seq + 1, bs).astype(np.int32)
        L[rep % bs] = q_len
        nc = (L - q_len).astype(np.int32)
        slots = np.concatenate([pt[i, (nc[i] + np.arange(q_len)) // P] * P
                                + (nc[i] + np.arange(q_len)) % P for i in range(bs)]).astype(np.int32)
        spec = dataclasses.replace(spec0, L=L, slot_mapping=slots)
        bits = lambda *shape: synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
        ht = synth.HostTensors(kp_host, vp_host, bits(T, Hq, 128), bits(T, Hkv, 128),
                               bits(T, Hkv, 128))
        nc_d.copy_(torch.from_numpy(nc))
        q_d.copy_(H.to_dev(spec, ht.q))
        k_d.copy_(H.to_dev(spec, ht.k))
        v_d.copy_(H.to_dev(spec, ht.v))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, _, kp_host, vp_host = oracle.store_then_attend(spec, ht, nthreads=8)
        assert np.array_equal(meta["seq_lens"].cpu().numpy(), L)
        assert np.array_equal(meta["slot_mapping"].cpu().numpy(), slots)
        assert np.array_equal(H.to_host_bits(spec, kpool), kp_host), f"replay {rep}: K pool"
        err = H.max_err(out_d, ref)
        assert err <= H.TOL["bf16"], f"replay {rep}: max abs err {err:.3e}"
        torch.ones(4096, device="cuda").mul_(2)  # eager work between replays


def test_graph_decode_capacity_checks():
    """Checked on the host before anything is enqueued."""
    import ctypes
    spec = uniform_batch("cap", 32, 8, 16, 1, 4, 500, np.random.default_rng(1))
    plan = graph_plan(spec, 4, 1, 500)
    f = ctypes.c_void_p(0x1000)
    call = lambda batch, cols: rp.lib.rpkv_graph_decode_forward(
        plan._h, batch, f, f, f, f, f, f, f, f, cols, cols, f, 0.1, None)
    assert call(5, 40) == 6                       # batch over capacity
    assert call(4, 31) == 1                       # too few page-table columns for 500 keys
    with pytest.raises(rp.RpkvError):
        plan.graph_decode_init(4, 5, 500)         # 5 tokens x G=4 rows > 16
