"""GPU parity for tiles cut every 128 (token, head) rows.

Where G = Hq / Hkv does not divide 128 and no tile of a prefill-type request is
key-split, its tiles hold 128 consecutive rows of the request's token-major
(token, head) rows, so a token's heads may straddle two tiles.  Each case below
mixes such requests with a long one whose tiles are key-split (and so stay
whole-token) and with decodes, and compares every output row with the fp64
oracle, for both tile arrangements; the store is compared bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests import gpu_harness as H
from workloads import synth

pytestmark = pytest.mark.gpu

CASES = [
    # name, Hq, Hkv, n, L
    ("g3", 24, 8, [300, 150, 1, 1, 77], [300, 1500, 900, 40, 77]),
    ("g5", 20, 4, [260, 130, 1, 2, 19], [260, 2000, 700, 600, 19]),
    ("g6", 12, 2, [211, 96, 1, 45], [211, 1300, 1000, 300]),
    ("g7", 28, 4, [512, 128, 1, 1], [512, 1800, 2000, 256]),
    ("g12", 24, 2, [101, 64, 1, 3], [101, 1100, 500, 200]),
    ("g24", 24, 1, [57, 40, 1, 2], [57, 1000, 333, 128]),
    ("g96", 96, 1, [9, 5, 1], [9, 900, 257]),
]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_row_cut_tiles_match_oracle(case):
    name, Hq, Hkv, n, L = case
    spec = synth.build(name, "bf16", Hq, Hkv, 128, 16, n, L, 31,
                       np.random.default_rng(zlib.crc32(name.encode())), 1.25)
    ht = synth.host_tensors(spec)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
    for tpb in (1, 2):
        db = H.dev_batch(spec, ht)
        out, plan = H.gpu_forward(spec, db, tiles_per_block=tpb)
        items = plan.items(0)
        assert ((items[:, 3] >> 16) > 0).any(), "no tile starts inside a token"
        assert (items[:, 7] >= 0).any(), "no key-split tile"
        assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref)
        assert np.array_equal(H.to_host_bits(spec, db.vpool), vp_ref)
        err = H.max_err(out, ref)
        print(f"{name} tpb={tpb}: max err {err:.2e}")
        assert err <= H.TOL[spec.dtype], (name, tpb, err)
