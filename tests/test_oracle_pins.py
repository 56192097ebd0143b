"""Pins for the fp64 oracle: what the pages and the mathematics fix, independent
of the oracle's own code.

* values the pages print (tests/golden/*.txt, each with its citation);
* the pages' own correctness check -- each request computed as complete causal
  attention on its contiguous sequence, keeping the last n rows -- done with
  torch's scaled_dot_product_attention in float64 (a library routine);
* closed forms (one key, zero query, ramp and needle probes);
* invariants (mixed pass == each request alone, decode row == last row of the
  full prefill, page relocation, poison of unreferenced slots, split/cascade
  merge == unsplit, GQA replication);
* a brute-force formulation with an explicit numpy mask matrix.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import synth
from tests import _golden


# ------------------------------------------------------------------ helpers

def make(n, L, P=4, Hq=4, Hkv=2, D=32, dtype="bf16", seed=0, pool_factor=1.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    spec = synth.build("t", dtype, Hq, Hkv, D, P, n, L, seed, rng, pool_factor)
    return spec, synth.host_tensors(spec)


def run(spec, t, **kw):
    out, lse, kp, vp = oracle.store_then_attend(spec, t, **kw)
    return out, lse, kp, vp


def logical_kv(spec, pool, i):
    """K (or V) of request i as its contiguous logical sequence [L, Hkv, D]."""
    slots = synth.request_slots(spec.page_table[i], int(spec.L[i]), spec.P)
    return synth.as_float64(spec, pool[slots])


def sdpa_reference(spec, t, kp, vp):
    """Complete causal attention of each request's whole sequence alone (float64,
    torch SDPA with is_causal and enable_gqa), keeping the last n rows."""
    cu = spec.cu_q
    outs = []
    g = torch.Generator().manual_seed(123)
    for i in range(spec.bs):
        n, L = int(spec.n[i]), int(spec.L[i])
        if n == 0:
            continue
        K = torch.from_numpy(logical_kv(spec, kp, i)).transpose(0, 1)  # [Hkv, L, D]
        V = torch.from_numpy(logical_kv(spec, vp, i)).transpose(0, 1)
        qn = torch.from_numpy(synth.as_float64(spec, t.q[cu[i]:cu[i + 1]]))  # [n, Hq, D]
        qfill = torch.randn(L - n, spec.Hq, spec.D, generator=g, dtype=torch.float64)
        Q = torch.cat([qfill, qn]).transpose(0, 1)  # [Hq, L, D]
        o = F.scaled_dot_product_attention(Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0),
                                           is_causal=True, scale=spec.scale, enable_gqa=True)
        outs.append(o[0].transpose(0, 1)[L - n:].numpy())
    return np.concatenate(outs) if outs else np.zeros((0, spec.Hq, spec.D))


# ------------------------------------------------------------------ golden values

def test_p1_worked_example_metadata():
    g = _golden.load("p1_worked_example.txt")
    rows = g["rows"]
    W = max(g["lens"])
    table = np.zeros((3, W), np.int32)
    for i, r in enumerate(rows):
        table[i, :len(r)] = r
    assert table.tolist() == g["page_table_cut"]
    n = [l - c for l, c in zip(g["lens"], g["cached"])]
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    assert cu.tolist() == g["cu_seqlens_q"]
    assert g["lens"] == g["cache_seqlens"]
    # this step's slots: positions cached..len-1 through each row
    out_loc = [oracle.slot(table, i, p, g["page_size"])
               for i in range(3) for p in range(g["cached"][i], g["lens"][i])]
    assert out_loc == g["out_loc"]
    assert oracle.last_indices(cu).tolist() == g["last_indices"]
    # the generator's slot lists agree with the oracle's slot rule on this example
    for i in range(3):
        assert synth.request_slots(table[i], g["lens"][i], 1).tolist() == rows[i]


@pytest.mark.parametrize("name", ["p5_layout.txt", "p5_mixed_step2.txt", "p5_exercise.txt"])
def test_p5_metadata(name):
    g = _golden.load(name)
    qsl, seq, pos, _, lg = oracle.build_batch(g["num_computed"], g["n"], g["need_logits"])
    assert qsl.tolist() == g["query_start_loc"]
    assert seq.tolist() == g["seq_lens"]
    assert pos.tolist() == g["positions"]
    assert lg.tolist() == g["logits_indices"]


def test_p1_cu_seqlens_forms():
    g = _golden.load("p1_cu_seqlens_forms.txt")
    lens = g["prefill_lens"]
    qsl, seq, _, _, _ = oracle.build_batch([0] * len(lens), lens, [1] * len(lens))
    assert qsl.tolist() == g["prefill_cu_seqlens_q"]
    assert np.concatenate([[0], np.cumsum(seq)]).tolist() == g["prefill_cu_seqlens_q"]
    bs = g["decode_bs"]
    qsl, _, _, _, lg = oracle.build_batch([7, 3, 9, 1], [1] * bs, [1] * bs)
    assert qsl.tolist() == g["decode_cu_seqlens_q"]
    assert lg.tolist() == list(range(bs))


def test_build_batch_slots_follow_block_tables():
    """slot of position x = table[x // P] * P + x % P, checked on a table whose
    entries are distinct, against the generator's listing of a row's slots."""
    P = 4
    tables = np.array([[7, 2, 9, 0], [5, 1, 3, 8]], np.int32)
    qsl, seq, pos, slots, _ = oracle.build_batch([3, 6], [6, 5], [1, 1], tables, P)
    want = np.concatenate([synth.request_slots(tables[0], 9, P)[3:9],
                           synth.request_slots(tables[1], 11, P)[6:11]])
    assert slots.tolist() == want.tolist()
    assert slots[0] == 7 * 4 + 3 and slots[1] == 2 * 4 + 0


def test_mask_rule_seven_keys_three_queries():
    g = _golden.load("p1_mask_rule.txt")
    L, n = g["kv_len"], g["n_queries"]
    spec, t = make([n], [L], P=1, Hq=2, Hkv=2, D=16, seed=3)
    base, _, kp, vp = run(spec, t)
    slots = synth.request_slots(spec.page_table[0], L, 1)
    for j in range(L):
        kp2, vp2 = kp.copy(), vp.copy()
        kp2[slots[j]] = synth.f32_to_bf16_bits(np.full(kp2[slots[j]].shape, 3.0, np.float32))
        vp2[slots[j]] = synth.f32_to_bf16_bits(np.full(vp2[slots[j]].shape, 5.0, np.float32))
        out, _ = oracle.attend(oracle.BF16, t.q, kp2, vp2, spec.page_table, spec.cu_q, spec.L,
                               2, 2, 16, 1, spec.scale)
        changed = [bool(np.any(out[r] != base[r])) for r in range(n)]
        for r in range(n):
            visible = j <= g["query_positions"][r]
            assert changed[r] == visible, (j, r)
        assert changed[0] == (j in g["first_query_visible"])


# ------------------------------------------------------------------ library routine

CASES = [
    # (n list, L list, P, Hq, Hkv)
    ([6, 3, 1], [6, 7, 9], 1, 4, 2),
    ([5, 1, 0, 9], [5, 17, 4, 33], 4, 4, 4),
    ([1, 1, 2], [40, 1, 2], 16, 8, 2),
    ([12, 3], [12, 29], 16, 4, 1),
    ([7], [23], 4, 6, 3),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_matches_complete_causal_attention(case, dtype):
    """The pages' own check: equal to each request's complete causal attention
    (no paging, no packing), last n rows, within fp64 rounding."""
    n, L, P, Hq, Hkv = case
    spec, t = make(n, L, P=P, Hq=Hq, Hkv=Hkv, D=32, dtype=dtype, seed=sum(L))
    out, lse, kp, vp = run(spec, t)
    ref = sdpa_reference(spec, t, kp, vp)
    assert out.shape == ref.shape
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_brute_force_explicit_mask_matrix():
    """Materialised [n, L] bottom-right mask (numpy tril with offset L-n) and a
    matrix softmax over the gathered keys, every small (n, L, P, G) combination."""
    for P in (1, 4, 16):
        for G in (1, 2, 4):
            for L in (1, 2, 3, 5, 8, 17, 40):
                for n in sorted({0, 1, 2, L}):
                    if n > L:
                        continue
                    Hkv = 2
                    Hq = Hkv * G
                    spec, t = make([n, 1], [L, 3], P=P, Hq=Hq, Hkv=Hkv, D=8, dtype="f32",
                                   seed=L * 97 + n * 7 + P + G)
                    out, _, kp, vp = run(spec, t)
                    K = logical_kv(spec, kp, 0)
                    V = logical_kv(spec, vp, 0)
                    mask = np.tril(np.ones((n, L), bool), k=L - n)
                    Q = t.q[:n].astype(np.float64)
                    for h in range(Hq):
                        S = spec.scale * Q[:, h, :] @ K[:, h // G, :].T
                        S = np.where(mask, S, -np.inf)
                        Pm = np.exp(S - S.max(axis=1, keepdims=True))
                        Pm /= Pm.sum(axis=1, keepdims=True)
                        np.testing.assert_allclose(out[:n, h], Pm @ V[:, h // G, :], rtol=0,
                                                   atol=1e-13)


# ------------------------------------------------------------------ closed forms

def test_single_key_returns_v():
    spec, t = make([1, 1], [1, 5], P=4, seed=5)
    out, _, kp, vp = run(spec, t)
    s = spec.slot_mapping[0]
    assert np.array_equal(out[0], np.repeat(synth.as_float64(spec, vp[s]), 2, axis=0))


def test_zero_query_gives_mean_of_visible_values():
    spec, t = make([4], [11], P=4, seed=6)
    t.q[:] = 0
    out, lse, kp, vp = run(spec, t)
    V = logical_kv(spec, vp, 0)
    for r in range(4):
        a = 11 - 4 + r
        for h in range(spec.Hq):
            np.testing.assert_allclose(out[r, h], V[:a + 1, h // spec.G].mean(axis=0), atol=1e-14)
            np.testing.assert_allclose(lse[r, h], np.log(a + 1), atol=1e-14)


def _ramp_inputs(spec, t, reverse=False):
    """K[x] = (x >> 8, x & 255, 0...) at logical position x (exact in bf16 for
    x < 32768), q = (256c, c, 0...) with c = 256, so q.K[x] = c*x exactly and the
    logits grow by c/sqrt(D) >= 20 per position."""
    c = 256.0
    kp, vp = t.kpool.copy(), t.vpool.copy()
    for i in range(spec.bs):
        slots = synth.request_slots(spec.page_table[i], int(spec.L[i]), spec.P)
        x = np.arange(int(spec.L[i]))
        Kx = np.zeros((len(x), spec.Hkv, spec.D), np.float32)
        Kx[:, :, 0] = (x >> 8)[:, None]
        Kx[:, :, 1] = (x & 255)[:, None]
        if reverse:
            Kx = -Kx
        kp[slots] = synth.f32_to_bf16_bits(Kx)
    q = np.zeros((spec.T, spec.Hq, spec.D), np.float32)
    q[:, :, 0] = 256 * c
    q[:, :, 1] = c
    return synth.f32_to_bf16_bits(q), kp, vp


@pytest.mark.parametrize("reverse", [False, True])
def test_ramp_probe_pins_every_row_boundary(reverse):
    n = [5, 1, 16, 3]
    L = [5, 300, 70, 19]
    spec, t = make(n, L, P=16, Hq=8, Hkv=2, D=128, seed=9)
    q, kp, vp = _ramp_inputs(spec, t, reverse)
    # no store: the probe fills every position of each row directly
    out, _ = oracle.attend(oracle.BF16, q, kp, vp, spec.page_table, spec.cu_q, spec.L,
                           spec.Hq, spec.Hkv, spec.D, spec.P, spec.scale)
    cu = spec.cu_q
    for i in range(spec.bs):
        V = logical_kv(spec, vp, i)
        for r in range(int(spec.n[i])):
            a = int(spec.L[i]) - int(spec.n[i]) + r
            want = V[0 if reverse else a]
            for h in range(spec.Hq):
                np.testing.assert_allclose(out[cu[i] + r, h], want[h // spec.G], atol=1e-6)


def test_needle_visible_iff_at_or_before_position():
    L, n = 50, 6
    spec, t = make([n], [L], P=4, Hq=2, Hkv=1, D=64, seed=4)
    kp0, vp0 = t.kpool.copy(), t.vpool.copy()
    oracle.store_kv(kp0, vp0, t.k, t.v, spec.slot_mapping)
    q = np.zeros((n, 2, 64), np.float32)
    q[:, :, 3] = 8.0
    q = synth.f32_to_bf16_bits(q)
    slots = synth.request_slots(spec.page_table[0], L, spec.P)
    for p in (0, 3, 4, 43, 44, 45, 46, 49):
        kp = kp0.copy()
        Kn = np.zeros((1, 64), np.float32)
        Kn[0, 3] = 64.0   # logit 8*64/8 = 64 against N(0,1)-free zeros elsewhere
        kp[slots[p]] = synth.f32_to_bf16_bits(Kn)
        out, _ = oracle.attend(oracle.BF16, q, kp, vp0, spec.page_table, spec.cu_q, spec.L, 2, 1,
                               64, spec.P, spec.scale)
        Vn = synth.as_float64(spec, vp0[slots[p], 0])
        for r in range(n):
            a = L - n + r
            hit = np.allclose(out[r, 0], Vn, atol=1e-9)
            assert hit == (p <= a), (p, r)


# ------------------------------------------------------------------ invariants

def test_mixed_pass_equals_each_request_alone():
    n = [9, 1, 0, 4, 1]
    L = [9, 33, 6, 21, 2]
    spec, t = make(n, L, P=4, Hq=4, Hkv=2, D=32, seed=21)
    out, lse, kp, vp = run(spec, t)
    cu = spec.cu_q
    for i in range(spec.bs):
        if n[i] == 0:
            continue
        sub_cu = np.array([0, n[i]], np.int32)
        o1, l1 = oracle.attend(oracle.BF16, t.q[cu[i]:cu[i + 1]], kp, vp, spec.page_table[i:i + 1],
                               sub_cu, spec.L[i:i + 1], 4, 2, 32, 4, spec.scale)
        assert np.array_equal(o1, out[cu[i]:cu[i + 1]])
        assert np.array_equal(l1, lse[cu[i]:cu[i + 1]])


def test_decode_row_equals_last_row_of_full_prefill():
    L = 37
    spec, t = make([L], [L], P=4, seed=31)
    out, _, kp, vp = run(spec, t)
    dec_cu = np.array([0, 1], np.int32)
    o1, _ = oracle.attend(oracle.BF16, t.q[L - 1:L], kp, vp, spec.page_table, dec_cu, spec.L, 4, 2,
                          32, 4, spec.scale)
    assert np.array_equal(o1[0], out[L - 1])


def test_page_relocation_leaves_output_unchanged():
    spec, t = make([3, 1, 8], [19, 26, 8], P=4, seed=41)
    out, _, kp, vp = run(spec, t)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(spec.num_pages).astype(np.int32)
    P = spec.P
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    for p in range(spec.num_pages):
        kp2[perm[p] * P:(perm[p] + 1) * P] = kp[p * P:(p + 1) * P]
        vp2[perm[p] * P:(perm[p] + 1) * P] = vp[p * P:(p + 1) * P]
    table2 = perm[spec.page_table]
    o2, _ = oracle.attend(oracle.BF16, t.q, kp2, vp2, table2, spec.cu_q, spec.L, 4, 2, 32, P,
                          spec.scale)
    assert np.array_equal(o2, out)


def test_poison_outside_rows_is_never_read():
    spec, t = make([3, 1, 8], [19, 26, 8], P=4, seed=42, pool_factor=3.0)
    out, _, kp, vp = run(spec, t)
    used = np.zeros(spec.num_slots, bool)
    for i in range(spec.bs):
        used[synth.request_slots(spec.page_table[i], int(spec.L[i]), spec.P)] = True
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[~used] = synth.f32_to_bf16_bits(np.zeros((1,), np.float32))[0]
    vp2[~used] = synth.f32_to_bf16_bits(np.full((1,), 8192.0, np.float32))[0]
    o2, _ = oracle.attend(oracle.BF16, t.q, kp2, vp2, spec.page_table, spec.cu_q, spec.L, 4, 2, 32,
                          4, spec.scale)
    assert np.array_equal(o2, out)


def test_gqa_head_map_is_consecutive_groups():
    """Hq=4 over Hkv=2 equals Hq=4 over Hkv=4 with KV heads replicated [0,0,1,1]:
    query head h uses KV head h // G (a map of h % Hkv would use [0,1,0,1])."""
    spec, t = make([5, 1], [12, 9], P=4, Hq=4, Hkv=2, D=32, seed=51)
    out, _, kp, vp = run(spec, t)
    kp4 = np.repeat(kp, 2, axis=1)
    vp4 = np.repeat(vp, 2, axis=1)
    o4, _ = oracle.attend(oracle.BF16, t.q, kp4, vp4, spec.page_table, spec.cu_q, spec.L, 4, 4, 32,
                          4, spec.scale)
    assert np.array_equal(o4, out)
    # and the alternative map really differs
    kpx = kp[:, [0, 1, 0, 1]]
    vpx = vp[:, [0, 1, 0, 1]]
    ox, _ = oracle.attend(oracle.BF16, t.q, kpx, vpx, spec.page_table, spec.cu_q, spec.L, 4, 4, 32,
                          4, spec.scale)
    assert not np.allclose(ox, out)


@pytest.mark.parametrize("bounds", [[0, 7, 20, 40, 70], [0, 16, 32, 48, 64, 70], [0, 1, 70],
                                    [0, 35, 35, 70]])
def test_split_keys_merge_equals_unsplit(bounds):
    """Disjoint key ranges attended apart and merged by log-sum-exp equal the
    unsplit result (split-KV decoding and the cascade's prefix/tail split)."""
    spec, t = make([1, 4, 1], [70, 66, 30], P=16, Hq=8, Hkv=2, D=64, seed=61)
    out, lse, kp, vp = run(spec, t)
    parts_o, parts_l = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        o, l = oracle.attend(oracle.BF16, t.q, kp, vp, spec.page_table, spec.cu_q, spec.L, 8, 2, 64,
                             16, spec.scale, key_lo=lo, key_hi=hi)
        parts_o.append(o.reshape(-1, 64))
        parts_l.append(l.reshape(-1))
    mo, ml = oracle.lse_merge(np.stack(parts_o), np.stack(parts_l))
    np.testing.assert_allclose(mo.reshape(out.shape), out, atol=1e-12, rtol=0)
    np.testing.assert_allclose(ml.reshape(lse.shape), lse, atol=1e-12, rtol=0)


def test_merge_of_empty_and_identical_parts():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((1, 3, 8))
    l = rng.standard_normal((1, 3))
    # two identical partials: same output, lse + ln 2
    mo, ml = oracle.lse_merge(np.concatenate([o, o]), np.concatenate([l, l]))
    np.testing.assert_allclose(mo, o[0], atol=1e-15)
    np.testing.assert_allclose(ml, l[0] + np.log(2), atol=1e-15)
    # an empty partial (lse = -inf, zero output) has no weight
    mo, ml = oracle.lse_merge(np.concatenate([o, np.zeros_like(o)]),
                              np.concatenate([l, np.full_like(l, -np.inf)]))
    assert np.array_equal(mo, o[0]) and np.array_equal(ml, l[0])
    # all empty: zero output, -inf lse, no NaN
    mo, ml = oracle.lse_merge(np.zeros((2, 3, 8)), np.full((2, 3), -np.inf))
    assert np.all(mo == 0) and np.all(ml == -np.inf)


def test_store_is_a_bitwise_scatter():
    spec, t = make([3, 2], [7, 9], P=4, seed=71)
    kp, vp = t.kpool.copy(), t.vpool.copy()
    sm = spec.slot_mapping.copy()
    sm[1] = -1   # a padded dummy token writes nothing
    oracle.store_kv(kp, vp, t.k, t.v, sm)
    want_k, want_v = t.kpool.copy(), t.vpool.copy()
    keep = sm >= 0
    want_k[sm[keep]] = t.k[keep]
    want_v[sm[keep]] = t.v[keep]
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v)


def test_store_before_attend_matters():
    """Attending before the store reads stale pool rows for this step's keys
    (exercise 2 of the reference backend page): the outputs differ."""
    spec, t = make([4, 1], [4, 9], P=4, seed=81)
    out, _, _, _ = run(spec, t)
    stale, _ = oracle.attend(oracle.BF16, t.q, t.kpool, t.vpool, spec.page_table, spec.cu_q,
                             spec.L, 4, 2, 32, 4, spec.scale)
    assert not np.allclose(stale, out)


def test_invalid_inputs_rejected():
    spec, t = make([2], [5], P=4, seed=1)
    with pytest.raises(ValueError):
        oracle.attend(oracle.BF16, t.q, t.kpool, t.vpool, spec.page_table,
                      np.array([0, 2], np.int32), np.array([1], np.int32), 4, 2, 32, 4, 0.1)
