"""GPU: rpkv_build_metadata (positions, query_start_loc, seq_lens, slot_mapping,
logits_indices built on the device) against the pages' printed examples and the
oracle's batch builder, bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_kv_store_amd as rp
from tests import _golden

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def dev(a, dtype=torch.int32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def run(nc, n, tables, P, need=None, max_tokens=None, out=None):
    o = rp.build_metadata(dev(nc), dev(n), dev(tables), P,
                          None if need is None else dev(need, torch.uint8), max_tokens, out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def check_against_oracle(nc, n, tables, P, need):
    B = len(nc)
    qsl, seq, pos, slots, lg = oracle.build_batch(nc, n, need, tables, P)
    got = run(nc, n, tables, P, need)
    N = int(np.sum(n))
    assert got["counts"][0] == N and got["counts"][1] == len(lg)
    assert np.array_equal(got["query_start_loc"][:B + 1], qsl)
    assert np.array_equal(got["seq_lens"][:B], seq)
    assert np.array_equal(got["positions"][:N], pos[:N])
    assert np.array_equal(got["slot_mapping"][:N], slots[:N])
    assert np.array_equal(got["logits_indices"][:len(lg)], lg)


@pytest.mark.parametrize("name", ["p5_layout.txt", "p5_mixed_step2.txt", "p5_exercise.txt"])
def test_printed_examples(name):
    g = _golden.load(name)
    nc, n, need = g["num_computed"], g["n"], g["need_logits"]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    tables = rng.permutation(4096)[:3 * 8].reshape(3, 8).astype(np.int32)
    got = run(nc, n, tables, 4, np.array(need, np.uint8))
    assert got["query_start_loc"][:4].tolist() == g["query_start_loc"]
    assert got["seq_lens"][:3].tolist() == g["seq_lens"]
    assert got["positions"][:len(g["positions"])].tolist() == g["positions"]
    m = len(g["logits_indices"])
    assert got["counts"][1] == m and got["logits_indices"][:m].tolist() == g["logits_indices"]
    check_against_oracle(np.array(nc), np.array(n), tables, 4, np.array(need, np.uint8))


def test_worked_example_slots():
    """The mini-sglang worked example (page size 1): out_loc are the slots."""
    g = _golden.load("p1_worked_example.txt")
    rows = g["rows"]
    tables = np.zeros((3, 9), np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = r
    nc = np.array(g["cached"], np.int32)
    n = np.array(g["lens"], np.int32) - nc
    got = run(nc, n, tables, 1)
    assert got["slot_mapping"][:10].tolist() == g["out_loc"]
    assert got["query_start_loc"].tolist() == g["cu_seqlens_q"]
    assert got["logits_indices"][:3].tolist() == g["last_indices"]


@pytest.mark.parametrize("seed,B,P", [(1, 1, 16), (2, 7, 1), (3, 300, 16), (4, 1024, 64),
                                      (5, 1025, 16), (6, 3000, 4), (7, 40, 1024)])
def test_random_batches_match_oracle(seed, B, P):
    rng = np.random.default_rng(seed)
    n = rng.integers(0, 40, B).astype(np.int32)
    n[rng.random(B) < 0.3] = 0
    n[rng.random(B) < 0.3] = 1
    nc = rng.integers(0, 500, B).astype(np.int32)
    cols = (int((nc + n).max()) + P - 1) // P + 1
    tables = rng.integers(0, 1 << 15, (B, cols + 3)).astype(np.int32)[:, :cols + 3]
    need = (rng.random(B) < 0.7).astype(np.uint8)
    check_against_oracle(nc, n, np.ascontiguousarray(tables), P, need)


def test_all_requests_need_logits_by_default():
    nc = np.array([3, 0, 9], np.int32)
    n = np.array([2, 0, 4], np.int32)
    tables = np.arange(30, dtype=np.int32).reshape(3, 10)
    got = run(nc, n, tables, 2)
    qsl, _, _, _, lg = oracle.build_batch(nc, n, np.ones(3, np.uint8), tables, 2)
    assert got["counts"][1] == 3 and np.array_equal(got["logits_indices"][:3], lg)


def test_tokens_past_capacity_not_written():
    nc = np.array([0, 5], np.int32)
    n = np.array([6, 4], np.int32)
    tables = np.arange(40, dtype=np.int32).reshape(2, 20)
    out = {"positions": torch.full((12,), -7, dtype=torch.int32, device="cuda"),
           "slot_mapping": torch.full((12,), -7, dtype=torch.int32, device="cuda")}
    got = run(nc, n, tables, 1, max_tokens=7, out=out)
    assert got["counts"][0] == 10
    assert got["positions"][:7].tolist() == [0, 1, 2, 3, 4, 5, 5]
    assert (got["positions"][7:] == -7).all() and (got["slot_mapping"][7:] == -7).all()


def test_graph_capture_and_replay():
    """Captured once, replayed with new inputs written in place; every replay
    matches the oracle (eager work and synchronisation between replays)."""
    B, P, cap = 64, 16, 64 * 40
    rng = np.random.default_rng(99)
    nc_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    n_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    tb_d = torch.zeros((B, 64), dtype=torch.int32, device="cuda")
    out = {k: torch.empty(sz, dtype=torch.int32, device="cuda") for k, sz in
           (("query_start_loc", B + 1), ("seq_lens", B), ("positions", cap),
            ("slot_mapping", cap), ("logits_indices", B), ("counts", 2))}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rp.build_metadata(nc_d, n_d, tb_d, P, max_tokens=cap, out=out, stream=s.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rp.build_metadata(nc_d, n_d, tb_d, P, max_tokens=cap, out=out,
                          stream=torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        n = rng.integers(0, 40, B).astype(np.int32)
        nc = rng.integers(0, 900, B).astype(np.int32)
        tb = rng.integers(0, 1 << 15, (B, 64)).astype(np.int32)
        nc_d.copy_(torch.from_numpy(nc))
        n_d.copy_(torch.from_numpy(n))
        tb_d.copy_(torch.from_numpy(tb))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        qsl, seq, pos, slots, lg = oracle.build_batch(nc, n, np.ones(B, np.uint8), tb, P)
        N = int(n.sum())
        got = {k: v.cpu().numpy() for k, v in out.items()}
        assert got["counts"].tolist() == [N, B]
        assert np.array_equal(got["query_start_loc"], qsl)
        assert np.array_equal(got["seq_lens"], seq)
        assert np.array_equal(got["positions"][:N], pos[:N])
        assert np.array_equal(got["slot_mapping"][:N], slots[:N])
        assert np.array_equal(got["logits_indices"][:B], lg)
        torch.zeros(1000, device="cuda").add_(1)  # eager work between replays
