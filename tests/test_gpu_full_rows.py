"""GPU parity at full size with dense row coverage.

The workloads at their stated sizes, in the launch configuration the benchmark
times (the planner's own choices), compared element by element with the fp64
oracle on many more rows than the sampled test: every row of the
Llama-3-8B-shaped mixed batch (the 2000-token prefill's every tile and key
split), every one of the 256 decodes of the decode-heavy batch, every row of one
512-token chunk over 4096 cached tokens plus every decode of the chunked-prefill
batch, and in the shared-prefix batch every
cascade member plus the first and last row of every 16-token tile of one
4096-token chunk over 28672 cached tokens.  The oracle runs on the sub-problem
of exactly the pages those requests reference, taken from the device before the
step's store; the store is compared bit for bit on those pages."""
import os

import numpy as np
import pytest
import torch

import oracle
from tests import gpu_harness as H
from workloads import synth

pytestmark = pytest.mark.gpu

# The oracle deals tokens to its threads round-robin; the sampled rows sit at
# 16-token tile edges, so an odd thread count spreads them over every thread.
THREADS = max(1, min(15, os.cpu_count() or 1))


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def run_dense(cid, reqs, rows_of):
    spec = synth.full_config(cid)
    db = H.device_contents(spec, seed=3000 + cid)
    sub = H.subproblem(spec, db, reqs)               # taken before the store
    rows = np.zeros(spec.T, bool)
    cu = spec.cu_q
    for i in reqs:
        for r in rows_of(spec, i):
            rows[cu[i] + r] = True
    sub_rows = rows[sub.token_map]
    out, plan = H.gpu_forward(spec, db)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(sub.spec, sub.tensors, rows=sub_rows,
                                                      nthreads=THREADS)
    got = H.to_f64(out[torch.from_numpy(sub.token_map).cuda()])
    err = float(np.abs(got[sub_rows] - ref[sub_rows]).max())
    print(f"{spec.name}: {int(sub_rows.sum())} rows x {spec.Hq} heads of {len(reqs)} requests, "
          f"max err {err:.2e}, plan {plan.info()}")
    assert err <= H.TOL[spec.dtype]
    P = spec.P
    pg = torch.from_numpy(sub.pages).cuda()
    kp = db.kpool.view(spec.num_pages, P, spec.Hkv, spec.D)[pg].reshape(-1, spec.Hkv, spec.D)
    vp = db.vpool.view(spec.num_pages, P, spec.Hkv, spec.D)[pg].reshape(-1, spec.Hkv, spec.D)
    assert np.array_equal(H.to_host_bits(spec, kp), kp_ref)
    assert np.array_equal(H.to_host_bits(spec, vp), vp_ref)
    assert bool(torch.isfinite(out.float()).all())
    return spec, plan


def every_row(spec, i):
    return range(int(spec.n[i]))


def test_llama3_8b_mixed_every_row():
    spec = synth.full_config(2)
    _, plan = run_dense(2, list(range(spec.bs)), every_row)
    # the long prefill's longest tiles are split by keys and merged
    assert plan.info()["num_merge_tokens"] > 6


def test_decode_heavy_every_decode():
    # the split-KV kernel in a launch of its own (K staged through LDS), every
    # one of the 256 decodes, most of them split into chunks and merged
    spec = synth.full_config(3)
    _, plan = run_dense(3, list(range(spec.bs)), every_row)
    info = plan.info()
    assert info["num_prefill_items"] == 0 and info["num_merge_tokens"] > spec.bs // 2


def test_chunked_prefill_one_chunk_and_every_decode():
    spec = synth.full_config(4)
    chunks = [i for i in range(spec.bs) if spec.n[i] > 1]
    decodes = [i for i in range(spec.bs) if spec.n[i] == 1]
    assert len(chunks) == 16 and len(decodes) == 32
    run_dense(4, [chunks[0]] + decodes, every_row)


def test_shared_prefix_members_and_every_tile_edge_of_one_chunk():
    spec = synth.full_config(5)
    members = [i for i in range(spec.bs) if spec.n[i] == 1]
    big = [i for i in range(spec.bs) if spec.n[i] > 1]
    assert len(members) == 64 and len(big) == 2
    tpt = 128 // spec.G                              # tokens per MFMA tile

    def rows(s, i):
        n = int(s.n[i])
        if n == 1:
            return [0]
        edges = set()
        for r0 in range(0, n, tpt):
            edges.update((r0, min(n, r0 + tpt) - 1))
        return sorted(edges)

    _, plan = run_dense(5, members + big[:1], rows)
    assert plan.info()["cascade_members"] == 64
