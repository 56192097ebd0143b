"""Shared-prefix tree of a batch's page-table rows -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the GPU library never does and shares no code with it.

What it follows (page title, then section):
  * SGLang source walkthrough "Attention backends", 3.2 "Page table": the radix
    cache turns the slots each request hits into the page-table tensors, so
    requests that reuse a cached prefix carry the same page ids for it;
  * same page, 3.3 "Cascade Inference": a prefix shared by several requests is
    attended once and merged with each request's own part by log-sum-exp, and the
    multi-level wrapper takes the radix tree's levels, one level per depth of
    sharing.

Readings (the pages give no construction; each is listed in the design notes):
  * a request may share a page only if every key of that page was cached before
    this step, so request j offers its first u_j = (L_j - n_j) // P page ids;
  * only eligible requests take part (the caller states which: the decode-type
    ones, whose new tokens all lie past any shared prefix);
  * the tree's nodes are the distinct classes "requests whose first k offered
    page ids agree", over every depth k >= 1, that hold at least two requests;
    a node's prefix is the deepest k that gives the same class, in keys k * P;
  * a node's parent is the smallest node that strictly contains it;
  * a level costs a pass and a merge term, so a node is kept only when it adds
    at least ``min_keys`` keys beyond its nearest kept ancestor (root: 0 keys);
    nodes are decided parents first.

Written as plain loops and dictionaries over small batches; no sorting tricks.
Parity status: pinned by tests/test_oracle_pins.py (a worked example derived by
hand and the pairwise longest-common-prefix characterisation).
"""
from __future__ import annotations

from typing import Dict, FrozenSet, List, Sequence


def offered_pages(L: int, n: int, P: int) -> int:
    """Pages of a request whose keys were all cached before this step."""
    return (int(L) - int(n)) // int(P)


def prefix_tree(rows, L: Sequence[int], n: Sequence[int], P: int, eligible: Sequence[bool],
                min_keys: int = 0) -> List[dict]:
    """Nodes of the shared-prefix tree, parents before children.

    rows: [bs, W] page ids (any int array-like); L, n: per-request KV length and
    new tokens; eligible: which requests take part.  Returns a list of dicts
    {"members": tuple of request indices (ascending), "prefix": keys,
    "parent": index into the list or -1}.
    """
    bs = len(L)
    E = [j for j in range(bs) if eligible[j]]
    offer = {j: [int(x) for x in list(rows[j])[:offered_pages(L[j], n[j], P)]] for j in E}

    # every class at every depth, with the deepest depth that yields it
    depth_of: Dict[FrozenSet[int], int] = {}
    max_k = max([len(v) for v in offer.values()], default=0)
    for k in range(1, max_k + 1):
        classes: Dict[tuple, List[int]] = {}
        for j in E:
            if len(offer[j]) >= k:
                classes.setdefault(tuple(offer[j][:k]), []).append(j)
        for members in classes.values():
            if len(members) >= 2:
                s = frozenset(members)
                depth_of[s] = max(depth_of.get(s, 0), k)

    # parents first: larger classes first; among equal sizes the order is free
    # (equal-size distinct classes are disjoint)
    sets = sorted(depth_of, key=lambda s: (-len(s), depth_of[s], sorted(s)))

    def parent_of(s):
        best = None
        for t in sets:
            if len(t) > len(s) and s < t and (best is None or len(t) < len(best)):
                best = t
        return best

    kept: Dict[FrozenSet[int], bool] = {}
    kept_anc: Dict[FrozenSet[int], object] = {}
    for s in sets:
        a = parent_of(s)
        while a is not None and not kept[a]:
            a = kept_anc[a]
        kept_anc[s] = a
        base = 0 if a is None else depth_of[a] * P
        kept[s] = depth_of[s] * P - base >= min_keys

    out_sets = [s for s in sets if kept[s]]
    index = {s: i for i, s in enumerate(out_sets)}
    return [{"members": tuple(sorted(s)), "prefix": depth_of[s] * P,
             "parent": -1 if kept_anc[s] is None else index[kept_anc[s]]} for s in out_sets]


def canonical(nodes: List[dict]):
    """Order-free form for comparisons: {(members, prefix, parent's members or ())}."""
    return {(tuple(nd["members"]), int(nd["prefix"]),
             tuple(nodes[nd["parent"]]["members"]) if nd["parent"] >= 0 else ())
            for nd in nodes}
