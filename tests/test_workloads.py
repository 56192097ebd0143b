"""Structure of the seeded synthetic batches (CPU only)."""
import numpy as np
import pytest

from workloads import synth


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("small", [False, True])
def test_batch_structure(cid, small):
    s = synth.small_config(cid) if small else synth.full_config(cid)
    assert np.all(s.n <= s.L) and np.all(s.n >= 0)
    assert s.cu_q[-1] == s.T == len(s.slot_mapping)
    assert s.Hq % s.Hkv == 0
    # slots referenced by different requests are disjoint, except a cascade group's
    # shared prefix; this step's slots are the last n positions of each row
    owner = {}
    shared = set()
    for (f, c, pl) in s.groups:
        shared |= set(synth.request_slots(s.page_table[f], pl, s.P).tolist())
    cu = s.cu_q
    for i in range(s.bs):
        sl = synth.request_slots(s.page_table[i], int(s.L[i]), s.P)
        assert sl.max() < s.num_slots
        assert len(set(sl.tolist())) == len(sl)
        for x in sl.tolist():
            if x in shared:
                continue
            assert owner.setdefault(x, i) == i
        assert np.array_equal(s.slot_mapping[cu[i]:cu[i + 1]], sl[int(s.L[i]) - int(s.n[i]):])
    assert len(set(s.slot_mapping.tolist())) == s.T
    for (f, c, pl) in s.groups:
        rows = s.page_table[f:f + c, :pl // s.P]
        assert np.all(rows == rows[0])
        # every member's new tokens lie beyond the shared prefix
        assert np.all(s.L[f:f + c] - s.n[f:f + c] >= pl)


def test_full_config_shapes():
    c2 = synth.full_config(2)
    assert c2.n.tolist() == [2000, 512, 1, 1, 1, 1, 1, 1]
    assert (c2.L[:2] == c2.n[:2]).all() and (c2.L[2:] >= 513).all() and (c2.L[2:] <= 4097).all()
    c3 = synth.full_config(3)
    assert c3.bs == 256 and (c3.L >= 1024).all() and (c3.L <= 8192).all()
    c4 = synth.full_config(4)
    assert (c4.n[:16] == 512).all() and (c4.L[:16] == 4608).all() and c4.Hq == 28 and c4.Hkv == 4
    c5 = synth.full_config(5)
    assert c5.groups == [(0, 64, 8192)] and (c5.L[64:] == 32768).all() and (c5.n[64:] == 4096).all()
    assert c5.Hq == 64 and c5.Hkv == 8


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0            # tie -> even
    assert back[2] == 1.0 + 2 ** -6  # tie -> even (upwards)
    assert back[3] == -2.5
