"""GPU: the alternate page-table formats.  FlashInfer's CSR form
(page_indices / page_indptr / last_page_len) must give exactly the plan and
outputs of the dense table it encodes; a block table rewritten into smaller
kernel pages must name the same slots (bit-exact against numpy) and give the
same attention."""
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


def to_csr(spec):
    pages = (spec.L + spec.P - 1) // spec.P
    indptr = np.concatenate(([0], np.cumsum(pages))).astype(np.int32)
    indices = np.concatenate([spec.page_table[i, :pages[i]] for i in range(spec.bs)] +
                             [np.zeros(0, np.int32)]).astype(np.int32)
    last = np.where(pages > 0, spec.L - (pages - 1) * spec.P, 0).astype(np.int32)
    return indptr, indices, last


def csr_forward(spec, db, host_copy=True, groups=None):
    indptr, indices, last = to_csr(spec)
    plan = H.make_plan(spec)
    idx_d = torch.from_numpy(indices if indices.size else np.zeros(1, np.int32)).cuda()
    plan.prepare_csr(spec.cu_q, indptr, last, idx_d, indices if host_copy else None,
                     spec.groups if groups is None else groups)
    out = torch.full_like(db.q, float("nan"))
    plan.forward(db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool, out, spec.scale)
    torch.cuda.synchronize()
    return out, plan


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("cid,host_copy", [(2, True), (3, False), (4, True), (5, True),
                                           (5, False), (1, True)])
def test_csr_equals_dense_table(cid, host_copy):
    spec = synth.small_config(cid)
    ht = synth.host_tensors(spec)
    ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    k0, v0 = db.kpool.clone(), db.vpool.clone()
    out_dense, p1 = H.gpu_forward(spec, db)
    db.kpool.copy_(k0)
    db.vpool.copy_(v0)
    out_csr, p2 = csr_forward(spec, db, host_copy)
    info1, info2 = p1.info(), p2.info()
    info1.pop("plan_host_us")
    info2.pop("plan_host_us")
    assert info1 == info2
    assert torch.equal(bits(out_dense), bits(out_csr))
    assert H.max_err(out_csr, ref) <= H.TOL[spec.dtype]


@pytest.mark.parametrize("case", [("page1", 1, [37, 1, 2], [37, 300, 70]),
                                  ("page64", 64, [200, 1, 0], [390, 1000, 5]),
                                  ("page256", 256, [3, 1], [700, 1500])])
def test_csr_edge_page_sizes(case):
    name, P, n, L = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    spec = synth.build(name, "bf16", 16, 4, 128, P, n, L, 7, rng, 1.3)
    ht = synth.host_tensors(spec)
    ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
    out, _ = csr_forward(spec, H.dev_batch(spec, ht))
    assert H.max_err(out, ref) <= H.TOL["bf16"]


def test_csr_rejects_bad_last_page_len():
    spec = synth.small_config(2)
    indptr, indices, last = to_csr(spec)
    last = last.copy()
    last[0] = spec.P + 1
    plan = H.make_plan(spec)
    with pytest.raises(rp.RpkvError):
        plan.prepare_csr(spec.cu_q, indptr, last, torch.from_numpy(indices).cuda())


@pytest.mark.parametrize("factor", [1, 2, 4, 16])
def test_rewrite_block_table_bit_exact(factor):
    rng = np.random.default_rng(factor)
    t = rng.integers(0, 1 << 20, (37, 53)).astype(np.int32)
    got = rp.rewrite_block_table(torch.from_numpy(t).cuda(), factor).cpu().numpy()
    want = (t[:, :, None] * factor + np.arange(factor)[None, None, :]).reshape(37, 53 * factor)
    assert np.array_equal(got, want)


def test_rewritten_table_gives_the_same_attention():
    """Cache blocks of 16 tokens, kernel pages of 4: the rewritten table names the
    same slots, so the output equals the 16-token-page run bit for bit."""
    spec = synth.small_config(2)
    ht = synth.host_tensors(spec)
    ref, _, _, _ = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    k0, v0 = db.kpool.clone(), db.vpool.clone()
    out16, _ = H.gpu_forward(spec, db)
    db.kpool.copy_(k0)
    db.vpool.copy_(v0)
    f = 4
    pt4 = rp.rewrite_block_table(db.page_table, f)
    spec4 = dataclasses.replace(spec, P=spec.P // f, num_pages=spec.num_pages * f,
                                page_table=pt4.cpu().numpy())
    db4 = dataclasses.replace(db, page_table=pt4)
    out4, _ = H.gpu_forward(spec4, db4)
    assert torch.equal(bits(out16), bits(out4))
    assert H.max_err(out4, ref) <= H.TOL["bf16"]
