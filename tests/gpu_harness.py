"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its C ABI, and build oracle sub-problems for sampled rows of
full-size batches.  Expected values always come from the oracle on the same
inputs; nothing here feeds GPU results to the oracle."""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
import ragged_paged_kv_store_amd as rp
from workloads import synth

TOL = {"bf16": 2e-2, "f32": 1e-4}


def torch_dtype(spec):
    return torch.bfloat16 if spec.dtype == "bf16" else torch.float32


def to_dev(spec, a: np.ndarray) -> torch.Tensor:
    if spec.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host_bits(spec, t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array in the oracle's encoding (uint16 bits / float32)."""
    if spec.dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.float().cpu().numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def make_plan(spec, **kw) -> rp.Plan:
    return rp.Plan(num_q_heads=spec.Hq, num_kv_heads=spec.Hkv, head_dim=spec.D, page_size=spec.P,
                   dtype=rp.BF16 if spec.dtype == "bf16" else rp.F32,
                   max_batch=max(spec.bs, 1), num_pages=spec.num_pages,
                   max_tokens=max(spec.T, 1), max_pages_per_req=max(spec.page_table.shape[1], 1),
                   **kw)


@dataclasses.dataclass
class DevBatch:
    kpool: torch.Tensor
    vpool: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    page_table: torch.Tensor
    slot_mapping: torch.Tensor


def dev_batch(spec, ht: synth.HostTensors) -> DevBatch:
    return DevBatch(to_dev(spec, ht.kpool), to_dev(spec, ht.vpool), to_dev(spec, ht.q),
                    to_dev(spec, ht.k), to_dev(spec, ht.v),
                    torch.from_numpy(np.ascontiguousarray(spec.page_table)).cuda(),
                    torch.from_numpy(np.ascontiguousarray(spec.slot_mapping)).cuda())


def gpu_forward(spec, db: DevBatch, groups=None, plan: Optional[rp.Plan] = None, **plan_kw):
    plan = plan or make_plan(spec, **plan_kw)
    plan.prepare(spec.cu_q, spec.L, db.page_table, spec.page_table,
                 spec.groups if groups is None else groups)
    out = torch.full_like(db.q, float("nan"))
    plan.forward(db.q, db.k, db.v, db.slot_mapping, db.kpool, db.vpool, out, spec.scale)
    torch.cuda.synchronize()
    return out, plan


def max_err(out_gpu: torch.Tensor, ref: np.ndarray, rows=None) -> float:
    got = to_f64(out_gpu)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.abs(got - ref).max())


# ---------------------------------------------------------------- full size

def device_contents(spec, seed: int) -> DevBatch:
    """N(0,1) contents drawn on the device with torch's seeded generator (the
    pools of the full-size batches are GBs; drawing them on the host is slow).
    bf16 values are the RNE conversion of fp32 draws."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = torch_dtype(spec)

    def fill(shape):
        t = torch.empty(shape, dtype=dt, device="cuda")
        flat = t.view(-1)
        step = 1 << 26
        for s in range(0, flat.numel(), step):
            e = min(flat.numel(), s + step)
            flat[s:e] = torch.randn(e - s, generator=g, device="cuda", dtype=torch.float32).to(dt)
        return t

    kpool = fill((spec.num_slots, spec.Hkv, spec.D))
    vpool = fill((spec.num_slots, spec.Hkv, spec.D))
    q = fill((spec.T, spec.Hq, spec.D))
    k = fill((spec.T, spec.Hkv, spec.D))
    v = fill((spec.T, spec.Hkv, spec.D))
    return DevBatch(kpool, vpool, q, k, v,
                    torch.from_numpy(np.ascontiguousarray(spec.page_table)).cuda(),
                    torch.from_numpy(np.ascontiguousarray(spec.slot_mapping)).cuda())


def pick_requests(spec, rng, max_reqs: int = 10) -> List[int]:
    bs = spec.bs
    cand = [0, bs - 1, int(np.argmax(spec.L)), int(np.argmin(spec.L)), int(np.argmax(spec.n))]
    for (f, c, _) in spec.groups:
        cand += [f, f + c - 1]
    cand += [int(x) for x in rng.choice(bs, size=min(bs, max_reqs), replace=False)]
    out = []
    for c in cand:
        if c not in out and spec.n[c] > 0:
            out.append(c)
    return sorted(out[:max_reqs])


def pick_rows(spec, reqs, rng, per_req: int = 6) -> np.ndarray:
    """Token rows to check: every row of short requests; for long ones the first
    and last rows, rows either side of 128/G-token tile edges and random rows."""
    cu = spec.cu_q
    sel = np.zeros(spec.T, bool)
    tpt = max(1, 128 // spec.G)
    for i in reqs:
        n = int(spec.n[i])
        if n <= per_req:
            sel[cu[i]:cu[i + 1]] = True
            continue
        rows = {0, n - 1, min(tpt, n - 1), min(tpt - 1, n - 1), n // 2}
        while len(rows) < per_req:
            rows.add(int(rng.integers(0, n)))
        for r in rows:
            sel[cu[i] + r] = True
    return sel


@dataclasses.dataclass
class SubProblem:
    spec: synth.BatchSpec
    tensors: synth.HostTensors
    reqs: List[int]
    token_map: np.ndarray   # sub token -> original token
    pages: np.ndarray       # original page ids, in sub-pool order


def subproblem(spec, db: DevBatch, reqs: Sequence[int]) -> SubProblem:
    """The chosen requests with only the pages they reference, renumbered, taken
    from the device BEFORE the step's store (the oracle performs the store)."""
    P = spec.P
    need = [spec.page_table[i, :-(-int(spec.L[i]) // P)] for i in reqs]
    pages = np.unique(np.concatenate(need)).astype(np.int64)
    remap = {int(p): j for j, p in enumerate(pages)}
    W = max(len(x) for x in need)
    table = np.zeros((len(reqs), W), np.int32)
    for r, x in enumerate(need):
        table[r, :len(x)] = [remap[int(p)] for p in x]
    cu = spec.cu_q
    tok = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in reqs])
    kp = db.kpool.view(spec.num_pages, P, spec.Hkv, spec.D)[torch.from_numpy(pages).cuda()]
    vp = db.vpool.view(spec.num_pages, P, spec.Hkv, spec.D)[torch.from_numpy(pages).cuda()]
    ti = torch.from_numpy(tok).cuda()
    sm = spec.slot_mapping[tok].astype(np.int64)
    sm_new = np.array([remap[int(s // P)] * P + int(s % P) for s in sm], np.int32)
    sub = synth.BatchSpec(name=spec.name + "_sub", dtype=spec.dtype, Hq=spec.Hq, Hkv=spec.Hkv,
                          D=spec.D, P=P, num_pages=len(pages),
                          n=spec.n[list(reqs)].copy(), L=spec.L[list(reqs)].copy(),
                          page_table=table, slot_mapping=sm_new, groups=[], seed=spec.seed)
    ht = synth.HostTensors(
        kpool=to_host_bits(spec, kp.reshape(-1, spec.Hkv, spec.D)),
        vpool=to_host_bits(spec, vp.reshape(-1, spec.Hkv, spec.D)),
        q=to_host_bits(spec, db.q[ti]), k=to_host_bits(spec, db.k[ti]),
        v=to_host_bits(spec, db.v[ti]))
    return SubProblem(sub, ht, list(reqs), tok, pages)
