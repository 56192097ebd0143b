#!/usr/bin/env python3
"""Benchmark: one batch step of ragged, paged, prefix-cached attention on one
MI355X, through the library's C ABI.

A step is the whole hot path for one batch of a 32-layer model: prepare_metadata
once (host planning + one upload), then for each layer forward(q, k, v, layer) =
store_kv of the step's K/V followed by attention (MFMA tiles, split-KV chunks,
log-sum-exp merge).  Each layer has its own q/k/v/out and KV pools; pools are
cycled so the working set between reuses exceeds the 256 MB Infinity Cache.
Inputs are seeded synthetic tensors already resident in HBM.

Default workload: the shared-prefix cascade batch, the largest of the five
(Hq=64, Hkv=8, D=128, page_size=16; 64 one-token decodes sharing an 8192-token
prefix with own tails uniform in [64, 1024], plus 2 chunked prefills of 4096 new
tokens over 28672 cached); value = algorithmic attention TFLOP/s (unmasked
query-key pairs x 4 x D x Hq) over the whole step.  The decode-heavy batch
(256 decodes, KV uniform in [1024, 8192]) is timed after it in the same run and
reported under extra.decode_heavy as KV-read GB/s with its own HBM roofline.
--workload picks another batch as the headline (the decode-heavy one reports
KV-read GB/s); --workload radix runs 128 decodes under a three-level
shared-prefix tree whose levels the planner finds from the page table each step,
and also times the same steps with the levels off.

Prints ONE JSON line (rank 0) with the roofline of the dominant kernel, measured
with HIP events on the launch stream in a second pass over the same steps, and
the fp64 CPU oracle timed on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
LAYERS = 32
METRIC = "attention TFLOP/s (prefill-heavy) and KV-read GB/s (decode-heavy), 1 MI355X"

WORKLOADS = {
    "c1": (1, "c1_tiny_mixed_fp32: query lens [6,3,1], KV [6,7,9], Hq=4 Hkv=2 D=64 page_size=1, fp32"),
    "c2": (2, "c2_llama3_8b_mixed: Hq=32 Hkv=8 D=128 page_size=16, query lens [2000,512,1x6], "
              "prefills uncached, decode history U[512,4096], bf16"),
    "c3": (3, "c3_decode_heavy: 256 decodes, KV U[1024,8192], Hq=32 Hkv=8 D=128 page_size=16, bf16"),
    "c4": (4, "c4_chunked_prefill: 16 x (4096 cached + 512 new) + 32 decodes KV U[256,2048], "
              "Hq=28 Hkv=4 D=128 page_size=16, bf16"),
    "c5": (5, "c5_shared_prefix_cascade: 64 decodes sharing an 8192-token prefix, tails U[64,1024], "
              "+ 2 x (28672 cached + 4096 new), Hq=64 Hkv=8 D=128 page_size=16, bf16"),
    "radix": (0, "radix_tree_decode: 128 decodes under a 3-level prefix tree (4096 keys shared "
                 "by all, 8 x 2048, 4 x 1024 per branch), tails U[64,512], shuffled order, "
                 "levels detected from the page table (>= 256 keys), Hq=32 Hkv=8 D=128 "
                 "page_size=16, bf16"),
}
RADIX_DETECT_KEYS = 256


def algorithmic(spec, tree):
    """Algorithmic work of one layer, split by kernel.

    flops = 4*D*Hq*sum over requests of [n(L-n) + n(n+1)/2] (unmasked pairs).
    KV bytes = 2*Hkv*D*b per unique slot read: a shared-prefix level's keys once
    for all its members.  `tree` is the plan's list of levels.
    """
    D, Hq, Hkv, b = spec.D, spec.Hq, spec.Hkv, spec.elem_bytes
    n = spec.n.astype(np.int64)
    L = spec.L.astype(np.int64)
    pairs = n * (L - n) + n * (n + 1) // 2
    G = spec.G
    dec = (n > 0) & (n * G <= 16)
    own_from = np.zeros(spec.bs, np.int64)   # first key of each request's own tail
    level_pairs = 0
    shared = 0                               # key reads the levels save
    for nd in tree:
        base = tree[nd["parent"]]["prefix"] if nd["parent"] >= 0 else 0
        seg = nd["prefix"] - base
        m = list(nd["members"])
        level_pairs += seg * int(n[m].sum())
        shared += seg * (len(m) - 1)
        own_from[m] = np.maximum(own_from[m], nd["prefix"])
    row_kv = 2 * Hkv * D * b
    flops_total = 4 * D * Hq * int(pairs.sum())
    flops_prefill = 4 * D * Hq * (int(pairs[~dec].sum()) + level_pairs)
    dec_keys = int((L - own_from)[dec].sum())
    kv_decode = row_kv * dec_keys
    kv_total = row_kv * (int(L.sum()) - shared)
    T = spec.T
    io = T * spec.Hq * D * b * 2 + T * Hkv * D * b * 2 * 2   # q read, out write, k/v read + pool write
    store_bytes = T * Hkv * D * b * 2 * 2
    return dict(flops_total=flops_total, flops_prefill=flops_prefill, kv_decode=kv_decode,
                kv_total=kv_total, bytes_total=kv_total + io, store_bytes=store_bytes,
                all_decode=bool(dec.all()))


def kernel_sources_hash() -> str:
    """Hash of the library's kernel and planner sources (as recorded in
    profiles/traffic.json when the HBM counters were taken)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "ragged_paged_kv_store_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(f).encode())
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by the copy calibration), or None when
    there is no such record or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(workload)
    if not k or k.get("kernel") != kernel or rec.get("source_hash") != kernel_sources_hash():
        return None
    return k["bytes_per_launch"]


def metadata_build_us(spec, db, rp, torch, reps: int = 50):
    """The batch's positions / query_start_loc / seq_lens / slot_mapping /
    logits_indices: built on the device (rpkv_build_metadata, HIP events around
    `reps` calls on the current stream) and, for comparison, vectorised with
    numpy on the host (an engine's usual build)."""
    nc = (spec.L - spec.n).astype(np.int32)
    n = spec.n.astype(np.int32)
    nc_d = torch.from_numpy(nc).cuda()
    n_d = torch.from_numpy(n).cuda()
    out = rp.build_metadata(nc_d, n_d, db.page_table, spec.P, max_tokens=max(spec.T, 1))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        rp.build_metadata(nc_d, n_d, db.page_table, spec.P, max_tokens=max(spec.T, 1), out=out)
    e1.record()
    torch.cuda.synchronize()
    dev_us = e0.elapsed_time(e1) * 1e3 / reps
    pt = spec.page_table
    t0 = time.perf_counter()
    for _ in range(reps):
        qsl = np.concatenate(([0], np.cumsum(n))).astype(np.int32)
        req = np.repeat(np.arange(spec.bs), n)
        pos = (nc[req] + np.arange(int(qsl[-1])) - qsl[:-1][req]).astype(np.int32)
        slots = pt[req, pos // spec.P] * spec.P + pos % spec.P
        seq = nc + n
        logits = qsl[1:] - 1
    host_us = (time.perf_counter() - t0) * 1e6 / reps
    del slots, seq, logits
    return {"device": round(dev_us, 2), "host_numpy": round(host_us, 2)}


def cpu_baseline(spec, db, H, budget_flops: float = 80e9):
    """The fp64 oracle as it stands, on the host, over one layer of the batch:
    every row when the layer is within ~80 GFLOP (about 30 core-seconds),
    otherwise a seeded sample of requests and rows within that budget, taken in
    runs of consecutive rows (the oracle deals consecutive tokens to its
    threads, so a run keeps every thread busy)."""
    import oracle
    from tests import gpu_harness as GH
    rng = np.random.default_rng(0)
    cores = min(16, os.cpu_count() or 1)
    n = spec.n.astype(np.int64)
    L = spec.L.astype(np.int64)
    layer_flops = 4 * spec.D * spec.Hq * int((n * (L - n) + n * (n + 1) // 2).sum())
    if layer_flops <= budget_flops:
        reqs = list(range(spec.bs))
        sub = GH.subproblem(spec, db, reqs)
        rows = np.ones(sub.spec.T, bool)
        sample = f"whole layer: all {spec.T} rows x {spec.Hq} heads"
    else:
        reqs = GH.pick_requests(spec, rng, max_reqs=16)
        sub = GH.subproblem(spec, db, reqs)
        s = sub.spec
        cu = s.cu_q
        rows = np.zeros(s.T, bool)
        acc = 0
        used = 0
        for i in rng.permutation(s.bs):
            ni, Li = int(s.n[i]), int(s.L[i])
            run = min(ni, cores)
            r0 = int(rng.integers(0, ni - run + 1))
            f = sum(4 * s.D * s.Hq * (Li - ni + r + 1) for r in range(r0, r0 + run))
            if acc + f > budget_flops and acc > 0:
                continue
            rows[cu[i] + r0:cu[i] + r0 + run] = True
            acc += f
            used += 1
        sample = (f"seeded sample: {int(rows.sum())} rows x {spec.Hq} heads of {used} requests, "
                  f"in runs of up to {cores} consecutive rows")
    s = sub.spec
    t0 = time.perf_counter()
    oracle.store_then_attend(s, sub.tensors, rows=rows, nthreads=cores)
    dt = time.perf_counter() - t0
    cu = s.cu_q
    flops = 0
    for i in range(s.bs):
        for r in range(int(s.n[i])):
            if rows[cu[i] + r]:
                flops += 4 * s.D * s.Hq * (int(s.L[i]) - int(s.n[i]) + r + 1)
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=sample + f", fp64, {dt:.2f} s wall", seconds=dt)


def setup(spec, layers, torch, H, tiles_per_block=0, prefix_detect_keys=0):
    """Per-layer device buffers of one workload: q/k/v/out for up to 8 layers and
    KV pool sets cycled so that more than 2 GB lies between reuses of a pool."""
    layer0 = H.device_contents(spec, seed=2024)
    pool_bytes = 2 * layer0.kpool.numel() * layer0.kpool.element_size()
    npools = int(min(layers, max(2, math.ceil(2e9 / pool_bytes))))
    pools = [(layer0.kpool, layer0.vpool)]
    for j in range(1, npools):
        d = H.device_contents(spec, seed=2024 + j)
        pools.append((d.kpool, d.vpool))
        del d
    qkv = [(layer0.q, layer0.k, layer0.v)]
    nq = min(layers, 8)
    for j in range(1, nq):
        g = torch.Generator(device="cuda")
        g.manual_seed(77 + j)
        dt = layer0.q.dtype
        qkv.append(tuple(torch.randn(t.shape, generator=g, device="cuda").to(dt)
                         for t in (layer0.q, layer0.k, layer0.v)))
    outs = [torch.empty_like(layer0.q) for _ in range(nq)]
    plan = H.make_plan(spec, prefix_detect_keys=prefix_detect_keys,
                       tiles_per_block=tiles_per_block)
    return dict(layer0=layer0, pools=pools, npools=npools, qkv=qkv, nq=nq, outs=outs, plan=plan)


def progress(msg):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def run_steps(step, steps, warmup, torch):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def roofline_of(dom, times, alg, decode_heavy):
    """Roofline of the dominant kernel from its HIP-event average duration."""
    n_l, ms_l = times[dom]
    avg_s = ms_l / n_l * 1e-3
    if dom == "fused" and decode_heavy:
        # decodes only: the launch streams every unique KV byte of the layer
        # (shared-prefix levels once, tails per request)
        roof = dict(bound="hbm", achieved=alg["kv_total"] / avg_s / 1e9, peak=PEAK_HBM_GBPS,
                    unit="GB/s")
    elif dom in ("prefill", "fused"):
        # the fused launch also streams the split-KV chunks; only the tiles'
        # algorithmic FLOPs are credited
        roof = dict(bound="mfma", achieved=alg["flops_prefill"] / avg_s / 1e12,
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s")
    elif dom == "decode":
        roof = dict(bound="hbm", achieved=alg["kv_decode"] / avg_s / 1e9, peak=PEAK_HBM_GBPS,
                    unit="GB/s")
    elif dom == "store":
        roof = dict(bound="hbm", achieved=alg["store_bytes"] / avg_s / 1e9, peak=PEAK_HBM_GBPS,
                    unit="GB/s")
    else:
        roof = dict(bound="alu", achieved=alg["flops_total"] / avg_s / 1e12, peak=78.6,
                    unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dom
    roof["avg_us"] = avg_s * 1e6
    return roof


def measure(workload, args, torch, rp, H, synth, cpu=True):
    """Time one workload: `args.steps` steps (prepare_metadata + layers x forward)
    after `args.warmup` untimed ones, then the same steps again with HIP events
    around every launch for the per-kernel averages and the roofline."""
    cid, desc = WORKLOADS[workload]
    layers = args.layers
    radix = workload == "radix"
    spec = synth.radix_tree() if radix else synth.full_config(cid)
    stream = torch.cuda.current_stream()
    progress(f"{workload}: drawing inputs")
    b = setup(spec, layers, torch, H, tiles_per_block=args.tiles_per_block,
              prefix_detect_keys=RADIX_DETECT_KEYS if radix else 0)
    progress(f"{workload}: {args.warmup} warm-up + {args.steps} timed steps of {layers} layers")
    layer0, pools, npools, qkv, nq, outs, plan = (b[k] for k in ("layer0", "pools", "npools",
                                                                 "qkv", "nq", "outs", "plan"))
    pt = layer0.page_table
    sm = layer0.slot_mapping
    # the radix workload's levels are found from the host page table each step
    pt_host = spec.page_table if radix else None

    def step():
        plan.prepare(spec.cu_q, spec.L, pt, pt_host, spec.groups, stream=stream)
        for l in range(layers):
            kp, vp = pools[l % npools]
            q, k, v = qkv[l % nq]
            plan.forward(q, k, v, sm, kp, vp, outs[l % nq], spec.scale, stream=stream)

    ms_per_step = run_steps(step, args.steps, args.warmup, torch)
    info = plan.info()
    progress(f"{workload}: {ms_per_step:.3f} ms per step; per-launch timing pass")

    # second pass over the same steps with HIP events around every launch
    plan.timing_enable(True, max_launches=8 * layers * args.steps + 64)
    for _ in range(args.steps):
        step()
    times = plan.timing_collect()
    plan.timing_enable(False)
    torch.cuda.synchronize()

    alg = algorithmic(spec, plan.cascade_tree())
    per_kernel = {k: {"launches": n, "avg_us": (ms * 1e3 / n) if n else None}
                  for k, (n, ms) in times.items()}
    decode_heavy = alg["all_decode"] and spec.dtype == "bf16"
    if decode_heavy:
        value = alg["kv_total"] * layers / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
    else:
        value = alg["flops_total"] * layers / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
    # dominant kernel: the one with the largest summed time
    dom = max((k for k in times if times[k][0]), key=lambda k: times[k][1])
    roof = roofline_of(dom, times, alg, decode_heavy)
    # counters were taken on the default run (32 layers, the planner's tile arrangement)
    roof["traffic"] = (measured_traffic(workload, dom)
                       if layers == LAYERS and args.tiles_per_block == 0 else None)

    flat = None
    if radix:
        # the same steps with the levels off: every request streams its whole prefix
        fplan = H.make_plan(spec)

        def fstep():
            fplan.prepare(spec.cu_q, spec.L, pt, None, [], stream=stream)
            for l in range(layers):
                kp, vp = pools[l % npools]
                q, k, v = qkv[l % nq]
                fplan.forward(q, k, v, sm, kp, vp, outs[l % nq], spec.scale, stream=stream)
        flat_ms = run_steps(fstep, args.steps, args.warmup, torch)
        flat = {"ms_per_step": round(flat_ms, 4), "speedup_with_levels": round(flat_ms / ms_per_step, 3),
                "kv_bytes_per_layer": int(algorithmic(spec, [])["kv_total"])}

    meta_us = metadata_build_us(spec, layer0, rp, torch)
    cpu_line = None
    if cpu:
        progress(f"{workload}: fp64 oracle on the host (cpu_baseline)")
        cpu_line = cpu_baseline(spec, layer0, H)
        cpu_line.pop("seconds", None)
        if unit == "GB/s":
            cpu_line["note"] = "oracle rate in TFLOP/s of the sampled rows"
    res = dict(
        desc=desc, spec=spec, value=value, unit=unit, ms_per_step=ms_per_step, roofline=roof,
        cpu_baseline=cpu_line, npools=npools,
        extra={
            "per_kernel": per_kernel,
            "layer_us": round(ms_per_step * 1e3 / layers, 2),
            "attention_tflops": round(alg["flops_total"] * layers / (ms_per_step * 1e-3) / 1e12, 3),
            "kv_read_GBps": round(alg["kv_total"] * layers / (ms_per_step * 1e-3) / 1e9, 1),
            "decode_kernel_GBps": (round(alg["kv_decode"] / (times["decode"][1] / times["decode"][0]
                                                             * 1e-3) / 1e9, 1)
                                   if times["decode"][0] else None),
            "split_kv_in_fused_launch": bool(times.get("fused", (0, 0))[0]),
            "algorithmic_per_layer": alg,
            "plan": info,
            "metadata_build_us": meta_us,
            "without_cascade_levels": flat,
            "cascade_tree": {"levels": info["num_cascade_levels"], "depth": info["cascade_depth"]},
        })
    del b, layer0, pools, qkv, outs, plan
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def graph_bench(args, torch, rp, H, synth):
    """--graph: the whole decode step (device metadata build + layers x
    graph-decode forward) captured in one HIP graph; its replays are timed."""
    cid, desc = WORKLOADS[args.workload]
    layers = args.layers
    spec = synth.full_config(cid)
    n0 = int(spec.n[0])
    if not (np.all(spec.n == n0) and n0 * spec.G <= 16 and spec.dtype == "bf16"):
        print("bench.py: --graph needs a uniform bf16 decode batch (e.g. --workload c3)",
              file=sys.stderr)
        sys.exit(2)
    b = setup(spec, layers, torch, H)
    layer0, pools, npools, qkv, nq, outs = (b[k] for k in ("layer0", "pools", "npools", "qkv",
                                                           "nq", "outs"))
    pt = layer0.page_table
    stream = torch.cuda.current_stream()
    gplan = H.make_plan(spec)
    max_seq = int(spec.L.max())
    gplan.graph_decode_init(spec.bs, n0, max_seq)
    nc_d = torch.from_numpy((spec.L - spec.n).astype(np.int32)).cuda()
    n_d = torch.from_numpy(spec.n.astype(np.int32)).cuda()
    meta = {k: torch.empty(sz, dtype=torch.int32, device="cuda") for k, sz in
            (("query_start_loc", spec.bs + 1), ("seq_lens", spec.bs), ("positions", spec.T),
             ("slot_mapping", spec.T), ("logits_indices", spec.bs), ("counts", 2))}
    gstream = torch.cuda.Stream()

    def gstep(st):
        rp.build_metadata(nc_d, n_d, pt, spec.P, max_tokens=spec.T, out=meta, stream=st)
        for l in range(layers):
            kp, vp = pools[l % npools]
            q, k, v = qkv[l % nq]
            gplan.graph_decode_forward(spec.bs, q, k, v, meta["slot_mapping"], kp, vp,
                                       meta["seq_lens"], pt, outs[l % nq], spec.scale,
                                       stream=st)

    with torch.cuda.stream(gstream):
        gstep(gstream.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gstream):
        gstep(torch.cuda.current_stream().cuda_stream)
    graph_ms = run_steps(graph.replay, args.steps, args.warmup, torch)
    # per-kernel durations of the same launches, eagerly, with HIP events
    gplan.timing_enable(True, max_launches=4 * layers * args.steps + 64)
    for _ in range(args.steps):
        gstep(stream.cuda_stream)
    gtimes = gplan.timing_collect()
    gplan.timing_enable(False)
    torch.cuda.synchronize()
    alg = algorithmic(spec, [])
    dec_n, dec_ms = gtimes["decode"]
    kv_rate = alg["kv_total"] * layers / (graph_ms * 1e-3) / 1e9
    avg_s = dec_ms / dec_n * 1e-3
    line = {
        "metric": METRIC,
        "value": round(kv_rate, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(graph_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) tensors, seeded page allocation)",
        "config": {"workload": desc, "layers_per_step": layers, "pool_sets": npools,
                   "batch": spec.bs, "tokens": spec.T,
                   "step": f"one HIP graph: device metadata build + {layers} x graph-decode "
                           "forward (store_kv + split-KV + merge)"},
        "roofline": {"bound": "hbm", "achieved": alg["kv_decode"] / avg_s / 1e9,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": alg["kv_decode"] / avg_s / 1e9 / PEAK_HBM_GBPS,
                     "kernel": "graph decode", "traffic": None},
        "cpu_baseline": None,
        "extra": {"per_kernel": {k: {"launches": nn, "avg_us": (ms * 1e3 / nn) if nn else None}
                                 for k, (nn, ms) in gtimes.items()},
                  "layer_us": round(graph_ms * 1e3 / layers, 2)},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS),
                    help="headline workload (default c5, the largest single-GPU batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-heavy", action="store_true",
                    help="skip the decode-heavy batch (c3) timed after the headline workload")
    ap.add_argument("--layers", type=int, default=LAYERS,
                    help="layers per step (a model has 32; fewer only for short profiling runs)")
    ap.add_argument("--graph", action="store_true",
                    help="uniform decode batches only: capture the whole step (device metadata "
                         "build + 32 graph-decode forwards) in one HIP graph and time its replays")
    ap.add_argument("--tiles-per-block", type=int, default=0, choices=[0, 1, 2],
                    help="MFMA tiles per workgroup (0: the planner's choice, as timed by "
                         "default; 1: one per 4-wavefront workgroup; 2: ping-pong pairs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU (asked for --gpus {args.gpus}); the "
              "path would shard by request or by KV head with no exchange between GPUs",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel(), "launches": 5}))
        return

    import ragged_paged_kv_store_amd as rp
    from tests import gpu_harness as H
    from workloads import synth

    if args.graph:
        graph_bench(args, torch, rp, H, synth)
        return

    r = measure(args.workload, args, torch, rp, H, synth, cpu=not args.no_cpu_baseline)
    spec = r["spec"]
    extra = r["extra"]
    # the decode-heavy batch in the same run: KV-read GB/s against the HBM roofline
    if args.workload != "c3" and not args.no_decode_heavy:
        d = measure("c3", args, torch, rp, H, synth, cpu=False)
        extra["decode_heavy"] = {
            "workload": d["desc"], "value": round(d["value"], 3), "unit": d["unit"],
            "ms_per_step": round(d["ms_per_step"], 4), "steps": args.steps,
            "warmup": args.warmup, "roofline": d["roofline"],
            "per_kernel": d["extra"]["per_kernel"], "layer_us": d["extra"]["layer_us"],
            "plan": d["extra"]["plan"],
        }
    line = {
        "metric": METRIC,
        "value": round(r["value"], 3),
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1) tensors, seeded page allocation)",
        "config": {"workload": r["desc"], "layers_per_step": args.layers,
                   "pool_sets": r["npools"], "batch": spec.bs, "tokens": spec.T,
                   "step": f"prepare_metadata + {args.layers} x (store_kv + attend)"},
        "roofline": r["roofline"],
        "cpu_baseline": r["cpu_baseline"],
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
