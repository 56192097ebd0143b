"""Seeded synthetic batches shaped like the workloads described on the pages.

This module only *builds inputs*: request lengths, page allocation from a shuffled
pool, each request's page-table row, the pool slots of this step's new tokens,
cascade hints, and tensor contents.  It contains none of the attention
arithmetic, so both the fp64 oracle and the GPU library can consume what it
produces without sharing any of the method's code.

Layout conventions (the boundary's, restated here because inputs must be built in
them):
  * queries are packed end to end: q[T, Hq, D]; request i owns rows
    [cu_q[i], cu_q[i+1]) (mini-sglang "The attention backend and a reference
    implementation", section "Variable-length, paged attention with prefixes");
  * the pool of one layer is K[num_pages, P, Hkv, D] and V of the same shape
    (the same page, section "The reference backend": the pool is flattened to
    [slots, Hkv, D]); slot s of page p and offset o is s = p*P + o;
  * a request's page-table row lists page ids; logical position x of request i
    lives in slot row[x // P]*P + x % P (block tables -> slot mapping, "Variable-
    length batching and one mixed forward pass", section "Layout and metadata");
  * this step's n new tokens are the last n logical positions [L-n, L).

Metadata draws from numpy's PCG64(seed): lengths, then the page permutation.
Contents draw from PCG64((seed, 1)): pool K, pool V, q, new k, new v, all
N(0,1).  bf16 tensors are round-to-nearest-even of fp32 draws.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np


@dataclasses.dataclass
class BatchSpec:
    """One batch's shape and metadata (all host numpy arrays)."""
    name: str
    dtype: str                      # "bf16" or "f32"
    Hq: int
    Hkv: int
    D: int
    P: int                          # page size in tokens
    num_pages: int
    n: np.ndarray                   # int32 [bs]  new tokens this step
    L: np.ndarray                   # int32 [bs]  KV length including this step
    page_table: np.ndarray          # int32 [bs, W] page ids, zero padded
    slot_mapping: np.ndarray        # int32 [T] pool slot of each new token
    groups: List[Tuple[int, int, int]]  # cascade hints (first_req, num_reqs, prefix_len)
    seed: int

    @property
    def bs(self) -> int:
        return int(self.n.shape[0])

    @property
    def cu_q(self) -> np.ndarray:
        cu = np.zeros(self.bs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.n, dtype=np.int64).astype(np.int32)
        return cu

    @property
    def T(self) -> int:
        return int(self.n.sum())

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.D))

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.P

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def request_slots(row: np.ndarray, length: int, P: int) -> np.ndarray:
    """Pool slots of logical positions 0..length-1 for one page-table row."""
    npages = -(-length // P)
    pages = row[:npages].astype(np.int64)
    return (np.repeat(pages * P, P) + np.tile(np.arange(P, dtype=np.int64), npages))[:length]


def _alloc_pages(rng, n_pages_each: List[int], shared: Optional[Tuple[List[int], int]],
                 pool_factor: float, P: int):
    """Allocate page ids consecutively from a seeded shuffle of the pool.

    shared = (member request indices, shared page count): those requests get the
    same first pages, allocated once.
    """
    unique = sum(n_pages_each)
    if shared is not None:
        members, sp = shared
        unique -= sp * (len(members) - 1)
    num_pages = max(int(np.ceil(unique * pool_factor)), 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    W = max(n_pages_each) if n_pages_each else 1
    table = np.zeros((len(n_pages_each), max(W, 1)), dtype=np.int32)
    cursor = 0
    shared_ids = None
    for i, npg in enumerate(n_pages_each):
        start = 0
        if shared is not None and i in shared[0]:
            sp = shared[1]
            if shared_ids is None:
                shared_ids = perm[cursor:cursor + sp].copy()
                cursor += sp
            table[i, :sp] = shared_ids
            start = sp
        need = npg - start
        table[i, start:npg] = perm[cursor:cursor + need]
        cursor += need
    assert cursor <= num_pages
    return table, num_pages


def build(name: str, dtype: str, Hq: int, Hkv: int, D: int, P: int, n, L, seed: int,
          rng: np.random.Generator, pool_factor: float,
          shared: Optional[Tuple[List[int], int]] = None, groups=None,
          table: Optional[np.ndarray] = None, num_pages: Optional[int] = None) -> BatchSpec:
    n = np.asarray(n, dtype=np.int32)
    L = np.asarray(L, dtype=np.int32)
    assert np.all(n <= L) and np.all(n >= 0)
    if table is None:
        n_pages_each = [int(-(-int(l) // P)) for l in L]
        shared_pages = None
        if shared is not None:
            assert shared[1] % P == 0, "a shared prefix covers whole pages"
            shared_pages = (shared[0], shared[1] // P)
        table, num_pages = _alloc_pages(rng, n_pages_each, shared_pages, pool_factor, P)
    slots = []
    for i in range(len(n)):
        s = request_slots(table[i], int(L[i]), P)
        slots.append(s[int(L[i]) - int(n[i]):])
    slot_mapping = (np.concatenate(slots) if slots else np.zeros(0)).astype(np.int32)
    return BatchSpec(name=name, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P, num_pages=int(num_pages),
                     n=n, L=L, page_table=table, slot_mapping=slot_mapping,
                     groups=list(groups or []), seed=seed)


# ----------------------------------------------------------------------------------
# The five workloads (full size) and their reduced twins used by the parity tests.
# ----------------------------------------------------------------------------------

def _u(rng, lo, hi, size):
    """Inclusive uniform integers."""
    return rng.integers(lo, hi + 1, size=size)


def c1_tiny(seed: int = 0) -> BatchSpec:
    """Worked example of the reference backend page: query lens [6,3,1], KV lens
    [6,7,9], Hq=4, Hkv=2, D=64, page_size=1, 64-slot pool, fp32; rows are disjoint
    slots from a seeded permutation."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n, L = [6, 3, 1], [6, 7, 9]
    perm = rng.permutation(64).astype(np.int32)
    table = np.zeros((3, max(L)), dtype=np.int32)
    c = 0
    for i, l in enumerate(L):
        table[i, :l] = perm[c:c + l]
        c += l
    return build("c1_tiny_mixed_fp32", "f32", 4, 2, 64, 1, n, L, seed, rng, 1.0,
                 table=table, num_pages=64)


def c2_llama8b_mixed(seed: int = 1, scale: float = 1.0) -> BatchSpec:
    """Llama-3-8B-shaped layer: query lens [2000,512,1x6]; prefills uncached;
    decodes with cached history uniform in [512,4096]; pool 1.25x."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pre = [max(int(2000 * scale), 1), max(int(512 * scale), 1)]
    hist = _u(rng, max(int(512 * scale), 1), max(int(4096 * scale), 1), 6)
    n = pre + [1] * 6
    L = pre + [int(h) + 1 for h in hist]
    return build("c2_llama3_8b_mixed" + ("" if scale == 1.0 else f"_x{scale}"), "bf16",
                 32, 8, 128, 16, n, L, seed, rng, 1.25)


def c3_decode_heavy(seed: int = 2, scale: float = 1.0, bs: int = 256) -> BatchSpec:
    """256 single-token decodes, KV length uniform in [1024,8192]; pool 1.1x."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = _u(rng, max(int(1024 * scale), 1), max(int(8192 * scale), 1), bs)
    n = [1] * bs
    return build("c3_decode_heavy" + ("" if scale == 1.0 else f"_x{scale}"), "bf16",
                 32, 8, 128, 16, n, L, seed, rng, 1.1)


def c4_chunked_prefill(seed: int = 3, scale: float = 1.0, n_pre: int = 16,
                       n_dec: int = 32) -> BatchSpec:
    """16 chunks of 512 new tokens over 4096 cached, plus 32 decodes with KV
    uniform in [256,2048]; Hq=28, Hkv=4; pool 1.25x."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cached, chunk = max(int(4096 * scale), 1), max(int(512 * scale), 1)
    Ld = _u(rng, max(int(256 * scale), 1), max(int(2048 * scale), 1), n_dec)
    n = [chunk] * n_pre + [1] * n_dec
    L = [cached + chunk] * n_pre + [int(x) for x in Ld]
    return build("c4_chunked_prefill" + ("" if scale == 1.0 else f"_x{scale}"), "bf16",
                 28, 4, 128, 16, n, L, seed, rng, 1.25)


def c5_shared_prefix(seed: int = 4, prefix: int = 8192, tail=(64, 1024), n_share: int = 64,
                     long_cached: int = 28672, long_new: int = 4096, n_long: int = 2,
                     name: str = "c5_shared_prefix_cascade") -> BatchSpec:
    """64 decodes sharing one 8192-token prefix (identical first 512 page ids),
    unique tails uniform in [64,1024] (L = prefix + tail, the decoded token being
    the last tail token), plus 2 chunked prefills of 4096 new tokens over 28672
    cached; Hq=64, Hkv=8; pool 1.1x of the unique pages."""
    rng = np.random.Generator(np.random.PCG64(seed))
    t = _u(rng, tail[0], tail[1], n_share)
    n = [1] * n_share + [long_new] * n_long
    L = [prefix + int(x) for x in t] + [long_cached + long_new] * n_long
    groups = [(0, n_share, prefix)] if n_share > 0 else []
    return build(name, "bf16", 64, 8, 128, 16, n, L, seed, rng, 1.1,
                 shared=(list(range(n_share)), prefix), groups=groups)


def radix_tree(seed: int = 5, bs: int = 128, levels=((1, 4096), (8, 2048), (4, 1024)),
               tail=(64, 512), shuffle: bool = True, Hq: int = 32, Hkv: int = 8, P: int = 16,
               extra_prefills=(), name: str = "radix_tree_decode", dtype: str = "bf16",
               D: int = 128) -> BatchSpec:
    """Decodes whose prefixes form a radix tree of shared pages (several sharing
    levels, as when a system prompt, per-task instructions and per-branch context
    are reused): level d splits every node of level d-1 into `fanout` children,
    each adding `keys` shared keys (a multiple of P).  The bs requests are dealt
    evenly to the leaves in tree order; each gets its own tail of U[tail] keys
    (the decoded token is the tail's last).  Every tree node's pages are allocated
    once from the shuffled pool (1.1x of the unique pages) and repeated in the rows
    of the requests under it.  shuffle=True permutes the request order, so members
    of a node are not contiguous; otherwise cascade hints (first_req, num_reqs,
    prefix_len) are returned for every node, nested.  extra_prefills: (cached,
    new) pairs appended as prefill-type requests with unshared pages."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nleaf = int(np.prod([f for f, _ in levels])) if levels else 1
    assert bs % nleaf == 0 and all(k % P == 0 for _, k in levels)
    per_leaf = bs // nleaf
    t = _u(rng, tail[0], tail[1], bs)
    n = [1] * bs + [int(b) for _, b in extra_prefills]
    L = [sum(k for _, k in levels) + int(x) for x in t] + [int(a) + int(b) for a, b in extra_prefills]
    # tree nodes in depth-first order: (depth, first request, count)
    nodes = []

    def walk(d, first, count):
        if d == len(levels):
            return
        f = levels[d][0]
        for c in range(f):
            sub = count // f
            nodes.append((d, first + c * sub, sub))
            walk(d + 1, first + c * sub, sub)
    walk(0, 0, bs)
    own = [-(-int(l) // P) for l in L]
    for (d, first, count) in nodes:
        for j in range(first, first + count):
            own[j] -= levels[d][1] // P
    unique = sum(levels[d][1] // P for d, _, _ in nodes) + sum(own)
    num_pages = max(int(np.ceil(unique * 1.1)), 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    W = max(-(-int(l) // P) for l in L)
    table = np.zeros((len(L), W), dtype=np.int32)
    fill = [0] * len(L)
    cursor = 0
    for (d, first, count) in nodes:
        np_ = levels[d][1] // P
        ids = perm[cursor:cursor + np_]
        cursor += np_
        for j in range(first, first + count):
            table[j, fill[j]:fill[j] + np_] = ids
            fill[j] += np_
    for j in range(len(L)):
        need = -(-int(L[j]) // P) - fill[j]
        table[j, fill[j]:fill[j] + need] = perm[cursor:cursor + need]
        cursor += need
    assert cursor <= num_pages
    prefix_at = np.cumsum([0] + [k for _, k in levels])
    groups = [(first, count, int(prefix_at[d + 1])) for (d, first, count) in nodes
              if count >= 1]
    if shuffle:
        order = np.concatenate([rng.permutation(bs), np.arange(bs, len(L))]).astype(np.int64)
        table = table[order]
        n = [n[i] for i in order]
        L = [L[i] for i in order]
        groups = []
    return build(name, dtype, Hq, Hkv, D, P, n, L, seed, rng, 1.1, groups=groups,
                 table=table, num_pages=num_pages)


def radix_tree_small(seed: int = 15, shuffle: bool = True, P: int = 16, Hq: int = 32,
                     Hkv: int = 8, extra_prefills=(), levels=None, dtype: str = "bf16",
                     D: int = 128) -> BatchSpec:
    """Reduced twin of radix_tree: 16 decodes, levels of 256 / 2x128 / 2x64 keys
    (scaled to the page size), tails U[5, 40]."""
    if levels is None:
        levels = ((1, max(256, 4 * P)), (2, max(128, 2 * P)), (2, max(64, P)))
    return radix_tree(seed=seed, bs=16, levels=levels, tail=(5, 40), shuffle=shuffle, Hq=Hq,
                      Hkv=Hkv, P=P, extra_prefills=extra_prefills,
                      name="radix_tree_decode_small", dtype=dtype, D=D)


def full_config(cid: int) -> BatchSpec:
    """The five workloads at their stated sizes (seeds 0..4)."""
    return {1: c1_tiny, 2: c2_llama8b_mixed, 3: c3_decode_heavy, 4: c4_chunked_prefill,
            5: c5_shared_prefix}[cid]()


def small_config(cid: int) -> BatchSpec:
    """Reduced twins of the five workloads: same structure (length mix, GQA ratio,
    page size, sharing), sizes the fp64 oracle finishes in seconds while still
    spanning several tiles, splits and a ragged tail."""
    if cid == 1:
        return c1_tiny()
    if cid == 2:
        return c2_llama8b_mixed(seed=11, scale=0.1)
    if cid == 3:
        return c3_decode_heavy(seed=12, scale=0.1, bs=24)
    if cid == 4:
        return c4_chunked_prefill(seed=13, scale=0.1, n_pre=3, n_dec=6)
    if cid == 5:
        return c5_shared_prefix(seed=14, prefix=640, tail=(6, 102), n_share=8,
                                long_cached=700, long_new=150, n_long=2,
                                name="c5_shared_prefix_cascade_small")
    raise ValueError(cid)


# ----------------------------------------------------------------------------------
# Tensor contents
# ----------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class HostTensors:
    """Tensor contents as host arrays: uint16 bf16 bit patterns or float32."""
    kpool: np.ndarray   # [num_slots, Hkv, D]
    vpool: np.ndarray
    q: np.ndarray       # [T, Hq, D]
    k: np.ndarray       # [T, Hkv, D]
    v: np.ndarray


def host_tensors(spec: BatchSpec, seed: Optional[int] = None) -> HostTensors:
    """N(0,1) contents drawn with numpy (small batches: the oracle reads these)."""
    # contents come from their own PCG64 stream keyed by (seed, 1), so that
    # changing a tensor's size never shifts the metadata draws
    rng = np.random.Generator(np.random.PCG64([spec.seed if seed is None else seed, 1]))
    conv = f32_to_bf16_bits if spec.dtype == "bf16" else (lambda a: a.astype(np.float32))
    shp_pool = (spec.num_slots, spec.Hkv, spec.D)
    kpool = conv(rng.standard_normal(shp_pool, dtype=np.float32))
    vpool = conv(rng.standard_normal(shp_pool, dtype=np.float32))
    q = conv(rng.standard_normal((spec.T, spec.Hq, spec.D), dtype=np.float32))
    k = conv(rng.standard_normal((spec.T, spec.Hkv, spec.D), dtype=np.float32))
    v = conv(rng.standard_normal((spec.T, spec.Hkv, spec.D), dtype=np.float32))
    return HostTensors(kpool, vpool, q, k, v)


def as_float64(spec: BatchSpec, a: np.ndarray) -> np.ndarray:
    if spec.dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)
