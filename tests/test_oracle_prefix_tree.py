"""Pins for the oracle's shared-prefix tree (oracle/prefix_tree.py).

* a worked example derived by hand from the definition (SGLang walkthrough
  "Attention backends", 3.2 and 3.3: requests that reuse a cached prefix carry its
  page ids; the multi-level cascade takes one level per depth of sharing), with
  the level pruning at several thresholds;
* on seeded random batches, the pairwise characterisation: the deepest node that
  holds two requests has exactly their longest common page prefix; a node's
  members are the requests whose common prefix with any member reaches the node's
  depth; nodes nest; every prefix is as deep as the members allow.
These statements use the pairwise longest common prefix, not the per-depth
classes the oracle enumerates.
"""
import itertools

import numpy as np

from oracle import prefix_tree as pt


def lcp_pages(a, b):
    k = 0
    while k < len(a) and k < len(b) and a[k] == b[k]:
        k += 1
    return k


# ------------------------------------------------------------ worked example
#
# page_size 2; every request decodes one token (n = 1).
#   req  row (page ids)   L   offered pages (L-1)//2   offered ids
#   0    5 6 7 8          9   4                        5 6 7 8
#   1    5 6 7 9          9   4                        5 6 7 9
#   2    5 6 3 4          8   3                        5 6 3
#   3    5 1 2 0          9   4                        5 1 2 0
#   4    5 6 7 8          3   1                        5
#   5    9 9 9 9          9   4                        9 9 9 9
#   6    5 6 7 8          9   -   not eligible (a prefill-type request)
# Classes of two or more: depth 1 {0,1,2,3,4} ("5"); depth 2 {0,1,2} ("5 6");
# depth 3 {0,1} ("5 6 7"); depth 4 has none.  Keys = 2 x depth.
# Unpruned tree: A={0..4} prefix 2, B={0,1,2} prefix 4 under A, C={0,1} prefix 6
# under B.
ROWS = np.array([[5, 6, 7, 8], [5, 6, 7, 9], [5, 6, 3, 4], [5, 1, 2, 0],
                 [5, 6, 7, 8], [9, 9, 9, 9], [5, 6, 7, 8]], np.int32)
L = [9, 9, 8, 9, 3, 9, 9]
N = [1, 1, 1, 1, 1, 1, 1]
ELIG = [True] * 6 + [False]
A, B, C = (0, 1, 2, 3, 4), (0, 1, 2), (0, 1)


def test_prefix_tree_worked_example_unpruned():
    got = pt.canonical(pt.prefix_tree(ROWS, L, N, 2, ELIG, 0))
    assert got == {(A, 2, ()), (B, 4, A), (C, 6, B)}


def test_prefix_tree_worked_example_pruned():
    # min 2 keys: every level adds 2 keys -> all kept
    assert pt.canonical(pt.prefix_tree(ROWS, L, N, 2, ELIG, 2)) == \
        {(A, 2, ()), (B, 4, A), (C, 6, B)}
    # min 3: A adds 2 -> dropped; B adds 4 over the root -> kept; C adds 2 over B
    assert pt.canonical(pt.prefix_tree(ROWS, L, N, 2, ELIG, 3)) == {(B, 4, ())}
    # min 4: same as 3 (B adds exactly 4)
    assert pt.canonical(pt.prefix_tree(ROWS, L, N, 2, ELIG, 4)) == {(B, 4, ())}
    # min 5: A, B dropped; C adds 6 over the root -> kept
    assert pt.canonical(pt.prefix_tree(ROWS, L, N, 2, ELIG, 5)) == {(C, 6, ())}
    # min 7: nothing adds 7 keys
    assert pt.prefix_tree(ROWS, L, N, 2, ELIG, 7) == []


def test_prefix_tree_new_tokens_not_offered():
    # request 0 with 3 new tokens over L=9 still offers (9-3)//2 = 3 pages "5 6 7":
    # the tree is unchanged
    n = list(N)
    n[0] = 3
    assert pt.canonical(pt.prefix_tree(ROWS, L, n, 2, ELIG, 0)) == \
        {(A, 2, ()), (B, 4, A), (C, 6, B)}
    # 4 new tokens: it offers (9-4)//2 = 2 pages "5 6"; C keeps one member and goes
    n[0] = 4
    assert pt.canonical(pt.prefix_tree(ROWS, L, n, 2, ELIG, 0)) == {(A, 2, ()), (B, 4, A)}
    # 6 new tokens: one page "5"; at depth 2 only requests 1 and 2 agree ("5 6")
    n[0] = 6
    assert pt.canonical(pt.prefix_tree(ROWS, L, n, 2, ELIG, 0)) == \
        {(A, 2, ()), ((1, 2), 4, A)}
    # 8 new tokens: no page offered; A loses request 0
    n[0] = 8
    assert pt.canonical(pt.prefix_tree(ROWS, L, n, 2, ELIG, 0)) == \
        {((1, 2, 3, 4), 2, ()), ((1, 2), 4, (1, 2, 3, 4))}


def test_prefix_tree_trivial_cases():
    assert pt.prefix_tree(np.zeros((0, 1), np.int32), [], [], 4, [], 0) == []
    # one request: no sharing
    assert pt.prefix_tree(np.array([[1, 2]]), [9], [1], 4, [True], 0) == []
    # two identical rows: one node at their whole offered length
    got = pt.prefix_tree(np.array([[1, 2, 3], [1, 2, 3]]), [12, 12], [1, 1], 4, [True, True], 0)
    assert pt.canonical(got) == {((0, 1), 8, ())}
    # differing first page: nothing
    assert pt.prefix_tree(np.array([[1, 2], [2, 2]]), [9, 9], [1, 1], 4, [True, True], 0) == []


# ------------------------------------------------ pairwise characterisation

def random_batch(rng, bs, width, alphabet):
    rows = rng.integers(0, alphabet, size=(bs, width)).astype(np.int32)
    # grow shared prefixes: copy a random other row's head into some rows
    for j in range(1, bs):
        if rng.random() < 0.7:
            src = int(rng.integers(0, j))
            k = int(rng.integers(0, width + 1))
            rows[j, :k] = rows[src, :k]
    P = int(rng.choice([1, 2, 4, 16]))
    n = rng.integers(0, 4, size=bs)
    L = np.array([int(rng.integers(max(int(n[j]), 1), max(int(n[j]), 1) + width * P + 1))
                  for j in range(bs)])
    elig = [bool(x) for x in rng.random(bs) < 0.85]
    return rows, L, n, P, elig


def test_prefix_tree_pairwise_characterisation():
    rng = np.random.Generator(np.random.PCG64(20251))
    for trial in range(60):
        bs = int(rng.integers(2, 14))
        rows, L, n, P, elig = random_batch(rng, bs, int(rng.integers(1, 7)), int(rng.integers(1, 4)))
        nodes = pt.prefix_tree(rows, L, n, P, elig, 0)
        E = [j for j in range(bs) if elig[j]]
        offer = {j: list(rows[j][:max(0, (int(L[j]) - int(n[j])) // P)]) for j in E}
        sets = [set(nd["members"]) for nd in nodes]
        # every pair: the smallest node holding both has their common prefix
        for i, j in itertools.combinations(E, 2):
            l = lcp_pages(offer[i], offer[j])
            holding = [k for k, s in enumerate(sets) if i in s and j in s]
            if l == 0:
                assert not holding, (trial, i, j)
            else:
                k = min(holding, key=lambda k: len(sets[k]))
                assert nodes[k]["prefix"] == l * P, (trial, i, j)
        for k, nd in enumerate(nodes):
            s, depth = sets[k], nd["prefix"] // P
            assert len(s) >= 2 and s <= set(E) and nd["prefix"] % P == 0 and depth >= 1
            m0 = nd["members"][0]
            # members: exactly the requests reaching this depth with a member
            assert s == {j for j in E if j == m0 or lcp_pages(offer[j], offer[m0]) >= depth}
            # as deep as the members allow: they do not all agree one page further
            deeper = [offer[j][:depth + 1] for j in s]
            assert any(len(x) <= depth for x in deeper) or len({tuple(x) for x in deeper}) > 1
            # nesting and the parent link
            for k2, s2 in enumerate(sets):
                if k2 != k:
                    assert not (s & s2) or s < s2 or s2 < s
            sup = [k2 for k2, s2 in enumerate(sets) if s < s2]
            if sup:
                par = min(sup, key=lambda k2: len(sets[k2]))
                assert nd["parent"] == par and nodes[par]["prefix"] < nd["prefix"]
                assert par < k   # parents first
            else:
                assert nd["parent"] == -1


def test_prefix_tree_pruning_threshold():
    """Kept levels add at least min_keys over their kept ancestor; a dropped level
    added fewer over the nearest kept ancestor of the unpruned tree."""
    rng = np.random.Generator(np.random.PCG64(7321))
    for trial in range(40):
        bs = int(rng.integers(2, 12))
        rows, L, n, P, elig = random_batch(rng, bs, int(rng.integers(2, 7)), 2)
        full = pt.prefix_tree(rows, L, n, P, elig, 0)
        mk = int(rng.integers(1, 4)) * P
        kept = pt.prefix_tree(rows, L, n, P, elig, mk)
        kept_sets = {nd["members"]: nd for nd in kept}
        for nd in kept:
            base = kept[nd["parent"]]["prefix"] if nd["parent"] >= 0 else 0
            assert nd["prefix"] - base >= mk
        for nd in full:
            # nearest kept ancestor within the unpruned tree
            a = nd["parent"]
            while a >= 0 and full[a]["members"] not in kept_sets:
                a = full[a]["parent"]
            base = full[a]["prefix"] if a >= 0 else 0
            assert (nd["members"] in kept_sets) == (nd["prefix"] - base >= mk), trial
