"""GPU parity on seeded random batches: random GQA ratio, KV heads, page size,
dtype, request mix (prefill, chunked prefill, decode, speculative decode, empty)
and split-KV tuning, each against the fp64 oracle on the same inputs (store
bit-exact, outputs within 2e-2 bf16 / 1e-4 fp32)."""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_harness as H
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def random_spec(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "f32" if seed % 4 == 3 else "bf16"
    G = int(rng.choice([1, 2, 4, 7, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4]))
    P = int(rng.choice([1, 4, 16, 64]))
    D = 128 if dtype == "bf16" else int(rng.choice([64, 128]))
    bs = int(rng.integers(1, 12))
    n, L = [], []
    for _ in range(bs):
        kind = int(rng.integers(0, 5))
        if kind == 0:      # prefill, nothing cached
            x = int(rng.integers(1, 300))
            n.append(x); L.append(x)
        elif kind == 1:    # chunked prefill over a cached prefix
            x = int(rng.integers(1, 200))
            n.append(x); L.append(x + int(rng.integers(1, 1500)))
        elif kind == 2:    # decode
            n.append(1); L.append(int(rng.integers(1, 3000)))
        elif kind == 3:    # a few new tokens (speculative decode)
            l = int(rng.integers(2, 2000))
            n.append(int(rng.integers(1, min(l, 4) + 1))); L.append(l)
        else:              # no new token this step
            n.append(0); L.append(int(rng.integers(0, 50)))
    spec = synth.build(f"random{seed}", dtype, G * Hkv, Hkv, D, P, n, L, seed,
                       np.random.default_rng(seed), 1.2)
    kw = dict(split_min_keys=int(rng.choice([0, 32, 64, 256])),
              split_target=int(rng.choice([0, 64, 512])))
    kw["tiles_per_block"] = int(rng.choice([0, 1, 2]))
    return spec, kw


@pytest.mark.parametrize("seed", range(256))
def test_random_batch_matches_oracle(seed):
    spec, kw = random_spec(seed)
    ht = synth.host_tensors(spec)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    out, plan = H.gpu_forward(spec, db, groups=[], **kw)
    assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref), "K pool differs after store"
    assert np.array_equal(H.to_host_bits(spec, db.vpool), vp_ref), "V pool differs after store"
    rows = np.ones(spec.T, bool)
    err = H.max_err(out, ref, rows) if spec.T else 0.0
    print(f"{spec.name}: G={spec.G} Hkv={spec.Hkv} P={spec.P} {spec.dtype} D={spec.D} "
          f"n={spec.n.tolist()} err {err:.2e} info {plan.info()}")
    assert err <= H.TOL[spec.dtype]


def random_decode_spec(seed):
    """A decode-only bf16 batch (every request has n * G <= 16 new rows), so the
    split-KV kernel runs in a launch of its own with K staged through LDS."""
    rng = np.random.default_rng(5000 + seed)
    G = int(rng.choice([1, 2, 4, 7, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    bs = int(rng.integers(1, 40))
    nmax = max(1, 16 // G)
    n, L = [], []
    for _ in range(bs):
        x = int(rng.integers(1, min(nmax, 3) + 1))
        n.append(x)
        L.append(x + int(rng.integers(0, int(rng.choice([40, 700, 6000])))))
    spec = synth.build(f"random_decode{seed}", "bf16", G * Hkv, Hkv, 128, P, n, L, seed,
                       np.random.default_rng(seed), 1.2)
    kw = dict(split_min_keys=int(rng.choice([0, 32, 64, 256])),
              split_target=int(rng.choice([0, 64, 512])))
    return spec, kw


@pytest.mark.parametrize("seed", range(96))
def test_random_decode_batch_matches_oracle(seed):
    spec, kw = random_decode_spec(seed)
    ht = synth.host_tensors(spec)
    ref, _, kp_ref, vp_ref = oracle.store_then_attend(spec, ht, nthreads=8)
    db = H.dev_batch(spec, ht)
    out, plan = H.gpu_forward(spec, db, groups=[], **kw)
    info = plan.info()
    assert info["num_prefill_items"] == 0 and info["num_decode_items"] > 0
    assert np.array_equal(H.to_host_bits(spec, db.kpool), kp_ref), "K pool differs after store"
    assert np.array_equal(H.to_host_bits(spec, db.vpool), vp_ref), "V pool differs after store"
    err = H.max_err(out, ref)
    print(f"{spec.name}: G={spec.G} Hkv={spec.Hkv} P={spec.P} n={spec.n.tolist()} "
          f"L={spec.L.tolist()} err {err:.2e} chunk {info['decode_chunk']}")
    assert err <= H.TOL["bf16"]
