#!/usr/bin/env python3
"""Benchmark of the multi-LoRA adapter path on one MI355X.

    python bench.py [--config decode|prefill|hetero|fused|fused_fp8|tiny|decode_qkv|prefill_qkv|decode_cache]
                    [--steps K] [--warmup W] [--paged PAGE_BYTES] [--graph] [--probe]

A step is one adapted layer-projection over one batch: shrink + expand for
every token (BGMV for the decode workload, SGMV from a prebuilt plan for the
others) or one fused call.  Steps rotate over L independent per-layer
instances (own adapters, activations and outputs) whose total footprint is at
least twice the 256 MB last-level cache, so timed calls read HBM as real
layers do.  Inputs are resident in HBM before timing starts.

Set-up (untimed): one step on every rotated instance (first touch of all
their memory), then W warmup steps; before each timed region a 512 MB read
evicts the last-level cache.  The timed region is exactly K steps issued one
library call at a time (each a prepared call whose arguments were converted
once); the same K steps recorded once as a HIP graph and replayed are timed
beside it (graph_ms_per_step; --graph makes that the reported figure).

Prints one JSON line: tokens/s per layer, ms per step, achieved algorithmic
HBM GB/s and its fraction of the 8 TB/s peak, the per-kernel durations and
their sum, the probes (empty launch, same-footprint stream, one dependent
round trip), a roofline object for the dominant kernel (its average duration
from HIP events that the library attaches to the kernel's own start and end,
on the launch stream) and the fp64 CPU oracle timed on the host cores
(cpu_baseline).  --probe prints the probe figures alone.
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, vendor figure
MALL_BYTES = 256 << 20

METRIC = "SGMV/BGMV tokens/s per layer + achieved HBM GB/s (% of MI355X peak)"
CONFIG_OF = {"tiny": 1, "decode": 2, "prefill": 3, "hetero": 4, "fused": 5, "fused_fp8": 5}


def algorithmic_bytes(prob):
    """Bytes the method must move for one layer: x once, each distinct adapter's
    A and B once (unpadded), y read + written once (written only when fused),
    W0 once (fused).  Returned per kernel: (shrink, expand, total)."""
    es = prob.esize
    distinct = prob.distinct_adapters()
    a_bytes = sum(int(prob.ranks[a]) * prob.d_in * es for a in distinct)
    b_bytes = sum(int(prob.ranks[a]) * prob.d_out * es for a in distinct)
    x_bytes = prob.T * prob.d_in * es
    if prob.meta.get("fused"):
        w_bytes = prob.d_out * prob.d_in * (1 if prob.W0_e4m3 is not None else es)
        y_bytes = prob.T * prob.d_out * es
        total = x_bytes + a_bytes + b_bytes + w_bytes + y_bytes
        return {"shrink": x_bytes + a_bytes, "fused": x_bytes + b_bytes + w_bytes + y_bytes, "total": total}
    n_adapted = int(np.count_nonzero(prob.ids >= 0))
    y_bytes = 2 * n_adapted * prob.d_out * es
    return {"shrink": x_bytes + a_bytes, "expand": b_bytes + y_bytes, "total": x_bytes + a_bytes + b_bytes + y_bytes}


def algorithmic_flops(prob, part="total"):
    """2 T sum r (d_in + d_out) for the adapters, plus 2 T d_in d_out for the
    base product when fused.  part="fused": the work of the fused GEMM kernel
    (base product and the B contraction; the x A shrink runs before it)."""
    ranks = [int(prob.ranks[a]) for a in prob.ids if a >= 0]
    if part == "fused":
        return 2 * prob.T * prob.d_in * prob.d_out + 2 * sum(ranks) * prob.d_out
    f = 2 * sum(r * (prob.d_in + prob.d_out) for r in ranks)
    if prob.meta.get("fused"):
        f += 2 * prob.T * prob.d_in * prob.d_out
    return f


class Instance:
    """One layer's worth of device-resident inputs, and its step as a
    prepared library call on the bench stream."""

    def __init__(self, prob, kind, stream, page_bytes=0, seed=0):
        import torch

        from segmented_gather_gemm_lora_amd import binding as B

        self.prob = prob
        self.kind = kind
        self.dt = prob.dtype
        self.page_bytes = page_bytes
        if page_bytes:
            # adapters in scattered frames of a page pool (seeded frame order)
            self.pool = B.PagedPool.from_problem(prob, page_bytes=page_bytes, shuffle_seed=seed)
        else:
            self.pool = B.DevicePool.from_problem(prob)
        self.x = B.to_device(prob.x, self.dt)
        self.y = B.to_device(prob.y_base(), self.dt)
        self.ids = torch.from_numpy(np.ascontiguousarray(prob.ids, dtype=np.int32)).cuda()
        self.plan = None
        if kind != "bgmv":
            self.plan = B.Plan(prob.T).build(prob.ids, self.pool).upload()
        op = {"bgmv": B.LORA_OP_BGMV, "sgmv": B.LORA_OP_SGMV}.get(kind)
        if op is not None:
            self.ws = B.workspace(op, prob.T, prob.d_in, prob.d_out, prob.max_rank)
        if kind == "fused":
            if prob.W0_e4m3 is not None:  # FP8 base: E4M3 codes, one byte each
                self.W0 = torch.from_numpy(np.ascontiguousarray(prob.W0_e4m3)).cuda()
            else:
                self.W0 = B.to_device(prob.W0, self.dt)
            nbytes = B.lora_workspace_bytes(B.LORA_OP_FUSED, prob.T, prob.d_in, prob.d_out, prob.max_rank)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        # the step: one library call with its arguments converted once
        if kind == "fused" and prob.W0_e4m3 is not None:
            self.step = B.fused_e4m3_prepared(self.x, self.W0, prob.w0_scale, self.plan, self.y, self.ws, stream)
        elif kind == "fused":
            self.step = B.fused_prepared(self.x, self.W0, self.plan, self.y, self.ws, self.dt, stream)
        elif kind == "bgmv":
            mk = B.bgmv_paged_prepared if page_bytes else B.bgmv_prepared
            self.step = mk(self.x, self.ids, self.pool, self.y, self.ws, self.dt, stream)
        elif page_bytes:
            self.step = B.sgmv_paged_prepared(self.x, self.plan, self.pool, self.y, self.ws, self.dt, stream)
        else:
            self.step = B.sgmv_prepared(self.x, self.plan, self.y, self.ws, self.dt, stream)


class GroupedInstance:
    """One layer's q, k, v inputs (shared x, own adapters and outputs) for the
    grouped call (BGMV for decode, SGMV from per-projection plans for
    prefill), and the same work as separate single calls, as prepared calls
    on the bench stream."""

    def __init__(self, probs, stream, sgmv=False):
        import torch

        from segmented_gather_gemm_lora_amd import binding as B

        self.sgmv = sgmv
        self.probs = probs
        dt = probs[0].dtype
        self.pools = [B.DevicePool.from_problem(p) for p in probs]
        self.x = B.to_device(probs[0].x, dt)
        self.ys = [B.to_device(p.y_base(), dt) for p in probs]
        self.ids = torch.from_numpy(np.ascontiguousarray(probs[0].ids, dtype=np.int32)).cuda()
        self.xs = [self.x] * len(probs)
        if sgmv:
            self.plans = [B.Plan(p.T).build(p.ids, pool).upload() for p, pool in zip(probs, self.pools)]
            self.projs = B.sgmv_proj_array(self.xs, self.plans, self.ys)
            self.ws = B.sgmv_grouped_workspace(self.projs)
            self.ws1 = [B.workspace(B.LORA_OP_SGMV, p.T, p.d_in, p.d_out, p.max_rank) for p in probs]
            self.step = B.sgmv_grouped_prepared(self.projs, self.ws, dt, stream, keep=(self.xs, self.plans, self.ys))
            sep = [B.sgmv_prepared(self.x, self.plans[p], self.ys[p], self.ws1[p], dt, stream)
                   for p in range(len(probs))]
        else:
            self.projs = B.proj_array(self.xs, self.pools, self.ys)
            self.ws = B.bgmv_grouped_workspace(probs[0].T, self.projs)
            self.ws1 = [B.workspace(B.LORA_OP_BGMV, p.T, p.d_in, p.d_out, p.max_rank) for p in probs]
            self.step = B.bgmv_grouped_prepared(probs[0].T, self.ids, probs[0].n_adapters, self.projs, self.ws, dt,
                                                stream, keep=(self.xs, self.pools, self.ys))
            sep = [B.bgmv_prepared(self.x, self.ids, self.pools[p], self.ys[p], self.ws1[p], dt, stream)
                   for p in range(len(probs))]

        def step_separate():
            for f in sep:
                f()

        self.step_separate = step_separate


def grouped_bytes(probs):
    """Algorithmic bytes of one grouped step: the shared x once, each
    projection's distinct adapters' A and B once, each y read and written once."""
    per = [algorithmic_bytes(p) for p in probs]
    x_bytes = probs[0].T * probs[0].d_in * probs[0].esize
    shrink = x_bytes + sum(a["shrink"] - x_bytes for a in per)
    expand = sum(a["expand"] for a in per)
    return {"shrink": shrink, "expand": expand, "total": shrink + expand}


FLUSH_BYTES = 512 << 20


class Timing:
    """Set-up, cache flush and the timed region of a benchmark on one stream.

    steps[i % L] is the step of rotated instance i.  Set-up runs every
    instance once and then W warmup steps; each timed region is preceded by a
    read of FLUSH_BYTES (twice the last-level cache) so that it starts with
    nothing of the workload cached."""

    def __init__(self, stream):
        import torch

        from segmented_gather_gemm_lora_amd import binding as B

        self.torch = torch
        self.B = B
        self.stream = stream
        self.flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(4096, dtype=torch.int32, device="cuda")

    def flush(self):
        B = self.B
        B._check(B.load().lora_probe_stream(self.stream.cuda_stream, self.flush_buf.data_ptr(), FLUSH_BYTES, None, 0,
                                            self.sink.data_ptr(), 2048), "lora_probe_stream")

    def setup(self, steps, W):
        for f in steps:
            f()
        for i in range(W):
            steps[i % len(steps)]()
        self.torch.cuda.synchronize()

    def eager(self, steps, K, first=0):
        """ms per step of K steps issued one call at a time, and the host wall time."""
        torch = self.torch
        L = len(steps)
        self.flush()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(self.stream)
        for i in range(K):
            steps[(first + i) % L]()
        ev1.record(self.stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / K, time.perf_counter() - t0

    def graph(self, steps, K, first=0):
        """ms per step of the same K steps recorded once as a graph and replayed
        (one untimed replay first), and the host wall time of the timed replay."""
        torch = self.torch
        L = len(steps)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(K):
                steps[(first + i) % L]()
        with torch.cuda.stream(self.stream):
            g.replay()
        torch.cuda.synchronize()
        self.flush()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(self.stream)
        with torch.cuda.stream(self.stream):
            g.replay()
        ev1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
        return ev0.elapsed_time(ev1) / K, wall

    def per_kernel(self, steps, names, K2):
        """Average duration of each kernel of a step (HIP events on the kernels
        themselves), over K2 eager steps; {name: us}."""
        torch, B = self.torch, self.B
        L = len(steps)
        nk = len(names)
        self.flush()
        torch.cuda.synchronize()
        timer = B.KernelTimer(K2 * nk)
        for i in range(K2):
            timer.arm(i * nk, nk)
            steps[i % L]()
        timer.disarm()
        torch.cuda.synchronize()
        out = {n: float(np.mean([timer.elapsed_us(i * nk + j) for i in range(K2)])) for j, n in enumerate(names)}
        timer.close()
        return out


def launches_per_step(step):
    """Kernels one library call enqueues (a probe step with events armed)."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    probe = B.KernelTimer(8)
    probe.arm(0, 8)
    step()
    used = B.KernelTimer.used()
    probe.disarm()
    torch.cuda.synchronize()
    probe.close()
    return used


def run_probes(stream, read_bytes, rmw_bytes, L, reps=200):
    """The achievable-at-this-size references: an empty launch back to back,
    one kernel moving the step's bytes (read_bytes read, rmw_bytes read and
    written back) rotating over L regions like the steps, and one dependent
    global-memory round trip.  Returns {name: us}."""
    import torch

    from segmented_gather_gemm_lora_amd import binding as B

    lib = B.load()
    sh = stream.cuda_stream
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    rd = (int(read_bytes) + 15) // 16 * 16
    rm = (int(rmw_bytes) + 15) // 16 * 16
    region = (rd + rm + 255) // 256 * 256
    buf = torch.zeros(region * L, dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, n):
        for i in range(min(n, 20)):
            fn(i)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(n):
            fn(i)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e3 / n

    out = {}
    out["empty_launch_us"] = timed(lambda i: B._check(lib.lora_probe_empty(sh, 1), "probe"), reps)
    out["empty_launch_1024wg_us"] = timed(lambda i: B._check(lib.lora_probe_empty(sh, 1024), "probe"), reps)
    base = buf.data_ptr()

    def stream_probe(i):
        r0 = base + (i % L) * region
        B._check(lib.lora_probe_stream(sh, r0, rd, r0 + rd, rm, sink.data_ptr(), 2048), "probe")

    n_stream = max(2 * L, min(reps, 20 * L))
    out["stream_same_bytes_us"] = timed(stream_probe, n_stream)
    out["stream_same_bytes_GBps"] = (rd + 2 * rm) / (out["stream_same_bytes_us"] * 1e-6) / 1e9
    # dependent loads 4 KB apart; run j follows its own chain (offset 64 j
    # bytes inside each 4 KB), so after the flush every load of a run misses
    # every cache
    stride, steps, runs = 1024, 2000, 5
    nxt = torch.zeros(stride * (steps + 1), dtype=torch.int32, device="cuda")
    k = torch.arange(steps, device="cuda", dtype=torch.int64)
    for j in range(runs):
        nxt[k * stride + 16 * j] = ((k + 1) * stride).to(torch.int32)
    assert int(nxt.max()) + 16 * runs < nxt.numel()
    Timing(stream).flush()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for j in range(runs):
        B._check(lib.lora_probe_chase(sh, nxt.data_ptr() + 64 * j, steps, sink.data_ptr()), "probe")
    ev[1].record(stream)
    torch.cuda.synchronize()
    out["dependent_load_us"] = ev[0].elapsed_time(ev[1]) * 1e3 / (runs * steps)
    del buf, nxt
    return {k: round(v, 3) for k, v in out.items()}


def grouped_main(args, stream, sgmv=False):
    """The q, k, v projections in one grouped call (one launch, or a shrink and
    an expand launch), with the same work as three single calls timed beside
    it: decode (BGMV) or, with sgmv, prefill (SGMV from per-projection plans)."""
    import torch

    from lora_workloads import PREFILL_QKV_NAME, QKV_NAME, make_decode_qkv, make_prefill_qkv

    make = make_prefill_qkv if sgmv else make_decode_qkv
    name = PREFILL_QKV_NAME if sgmv else QKV_NAME
    kind = "sgmv" if sgmv else "bgmv"
    probs0 = make()
    ab0 = grouped_bytes(probs0)
    L = args.rotation or rotation_count(ab0["total"])
    print(f"[bench] {name}: T={probs0[0].T} d_in={probs0[0].d_in} d_out={[p.d_out for p in probs0]} "
          f"rotation={L} bytes/layer={ab0['total']/1e6:.2f} MB", file=sys.stderr, flush=True)
    insts = [GroupedInstance(probs0, stream, sgmv)] + [GroupedInstance(make(seed=2000 + i), stream, sgmv)
                                                       for i in range(1, L)]
    torch.cuda.synchronize()
    ab_all = [grouped_bytes(g.probs) for g in insts]
    bytes_step = float(np.mean([a["total"] for a in ab_all]))
    T = probs0[0].T
    K = args.steps if args.steps is not None else 20 * L
    W = args.warmup if args.warmup is not None else 10 * L
    steps = [g.step for g in insts]
    sep = [g.step_separate for g in insts]
    tm = Timing(stream)
    tm.setup(steps, W)
    tm.setup(sep, 0)
    ms_step, t_wall, mode, other_ms, graph_note = timed_steps(tm, steps, K, W, args.graph)
    ms_sep, _, _, _, _ = timed_steps(tm, sep, K, W, args.graph)
    used = launches_per_step(steps[0])
    names = [kind] if used == 1 else ["shrink", "expand"]  # one launch: shrink and expand in one kernel
    assert len(names) == used, (names, used)
    per_kernel_us = tm.per_kernel(steps, names, max(L, min(K, 20 * L)))
    dominant = max(names, key=lambda n: per_kernel_us[n])
    if names == [kind]:
        for a in ab_all:
            a[kind] = a["total"]
    dom_bytes = float(np.mean([a[dominant] for a in ab_all]))
    dom_us = per_kernel_us[dominant]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic, kname = recorded_traffic(name, dominant)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "kernel": kname or (f"{kind}_grouped_onepass_kernel" if names == [kind] else
                                f"{kind}_{dominant}_grouped_kernel"),
            "algorithmic_bytes_per_launch": round(dom_bytes),
            "avg_launch_us": round(dom_us, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        cores = max(1, min(HOST_CORES, os.cpu_count() or 1))
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_budget:
            for p in probs0:
                oracle.lora_forward(p, nthreads=cores)
            reps += 1
        el = time.perf_counter() - t0
        cpu = {"value": reps * T / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"{reps} full q/k/v layers of {T} tokens ({el:.1f} s, fp64, OpenMP over tokens)",
               "host_nproc": os.cpu_count(), "cpu_model": cpu_model()}

    gbps = bytes_step / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": probs0[0].dtype,
        "data": "synthetic",
        "config": {"workload": name, "T": T, "d_in": probs0[0].d_in, "d_out": [p.d_out for p in probs0],
                   "ranks": [16], "pool_adapters": probs0[0].n_adapters,
                   "distinct_adapters": int(len(probs0[0].distinct_adapters())), "rotated_instances": L,
                   "path": f"{kind}_grouped"},
        "timed_mode": mode,
        ("graph_ms_per_step" if mode == "eager" else "eager_ms_per_step"):
            None if other_ms is None else round(other_ms, 6),
        "achieved_GBps": round(gbps, 1),
        "hbm_peak_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": round(bytes_step),
        "per_kernel_us": {n: round(v, 3) for n, v in per_kernel_us.items()},
        "kernel_sum_us": round(sum(per_kernel_us.values()), 3),
        "separate_calls_ms_per_step": round(ms_sep, 6),
        "separate_calls": f"the same q, k, v work as three lora_{kind} calls "
                          f"({launches_per_step(sep[0])} launches)",
        "wall_s_timed": round(t_wall, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if graph_note:
        out["graph_note"] = graph_note
    print(json.dumps(out))


def cache_main(args, stream):
    """Decode batches whose adapters come through the residency cache: 256
    adapters of rank 16 in pinned host memory, Zipf(1.1) popularity, a cache
    of 64 adapters; a step is lora_cache_prepare (copies of missing adapters on
    a copy stream) + one BGMV call.  The same batches with every adapter
    resident are timed beside it."""
    import torch

    import oracle
    from lora_workloads import CACHE_NAME, make_decode_registry
    from segmented_gather_gemm_lora_amd import binding as B

    prob, batches = make_decode_registry()
    n, T, slots = prob.n_adapters, prob.T, 64
    nb = len(batches)
    print(f"[bench] {CACHE_NAME}: T={T} registry={n} cache={slots} adapters, {nb} batches", file=sys.stderr,
          flush=True)
    ext = lambda r: (r * prob.d_in * 2 + 255) // 256 * 256 + (prob.d_out * r * 2 + 255) // 256 * 256  # noqa: E731
    buf = torch.zeros(B.load().lora_cache_table_bytes(n) + slots * ext(16), dtype=torch.uint8, device="cuda")
    cache = B.AdapterCache(buf, n, "bf16", prob.d_in, prob.d_out)
    for a in range(n):
        r = int(prob.ranks[a])
        A = torch.from_numpy(prob.pool[prob.a_off[a]: prob.a_off[a] + r * prob.d_in].copy()).pin_memory()
        Bm = torch.from_numpy(prob.pool[prob.b_off[a]: prob.b_off[a] + prob.d_out * r].copy()).pin_memory()
        cache.register(a, A, Bm, r, float(prob.alphas[a]))
    resident = B.DevicePool.from_problem(prob)
    x = B.to_device(prob.x, "bf16")
    y = B.to_device(prob.y_base(), "bf16")
    ids_dev = [torch.from_numpy(b).cuda() for b in batches]
    ws = B.workspace(B.LORA_OP_BGMV, T, prob.d_in, prob.d_out, 16)
    copy_stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    cache.prepare(batches[0], copy_stream, stream)
    cpool = cache.pool()  # device tables keep their addresses; host mirrors are not needed for BGMV

    def step_cache(i):
        cache.prepare(batches[i % nb], copy_stream, stream)
        B.bgmv(x, ids_dev[i % nb], cpool, y, ws, "bf16", max_rank=16, stream=stream)

    def step_resident(i):
        B.bgmv(x, ids_dev[i % nb], resident, y, ws, "bf16", max_rank=16, stream=stream)

    K = args.steps if args.steps is not None else 4 * nb
    W = args.warmup if args.warmup is not None else nb
    for i in range(W):
        step_cache(i)
        step_resident(i)
    torch.cuda.synchronize()
    tm = Timing(stream)
    s0 = cache.stats()
    ms_cache, t_wall = tm.eager([lambda i=i: step_cache(i) for i in range(nb)], K)
    s1 = cache.stats()
    ms_res, _ = tm.eager([lambda i=i: step_resident(i) for i in range(nb)], K)
    misses = (s1["misses"] - s0["misses"]) / K
    h2d = (s1["bytes_copied"] - s0["bytes_copied"]) / K
    hits = (s1["hits"] - s0["hits"]) / K

    timer = B.KernelTimer(2 * nb)
    for i in range(nb):
        timer.arm(2 * i, 2)
        step_cache(i)
    timer.disarm()
    torch.cuda.synchronize()
    per_kernel_us = {nm: float(np.mean([timer.elapsed_us(2 * i + j) for i in range(nb)]))
                     for j, nm in enumerate(["shrink", "expand"])}
    timer.close()
    dominant = max(per_kernel_us, key=per_kernel_us.get)
    dom_bytes = float(np.mean([algorithmic_bytes(dataclasses_replace_ids(prob, b))[dominant] for b in batches]))
    achieved = dom_bytes / (per_kernel_us[dominant] * 1e-6) / 1e9
    traffic, kname = recorded_traffic(CACHE_NAME, dominant)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "kernel": kname or f"bgmv_{dominant}", "algorithmic_bytes_per_launch": round(dom_bytes),
            "avg_launch_us": round(per_kernel_us[dominant], 3)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(prob, args.cpu_budget)
    out = {
        "metric": METRIC,
        "value": round(T / (ms_cache * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_cache, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": CACHE_NAME, "T": T, "d_in": prob.d_in, "d_out": prob.d_out, "ranks": [16],
                   "registry_adapters": n, "cache_adapters": slots, "popularity": "zipf 1.1", "batches": nb,
                   "path": "lora_cache_prepare + bgmv"},
        "resident_ms_per_step": round(ms_res, 6),
        "resident": "the same batches with all 256 adapters resident (no cache)",
        "misses_per_step": round(misses, 2),
        "hits_per_step": round(hits, 2),
        "h2d_bytes_per_step": round(h2d),
        "h2d_GBps_over_step": round(h2d / (ms_cache * 1e-3) / 1e9, 2),
        "per_kernel_us": {nm: round(v, 3) for nm, v in per_kernel_us.items()},
        "wall_s_timed": round(t_wall, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    cache.close()
    print(json.dumps(out))


def dataclasses_replace_ids(prob, ids):
    import dataclasses

    return dataclasses.replace(prob, ids=np.asarray(ids, dtype=np.int32))


def base_gemm_reference_us(inst, stream, reps=50):
    """Average time of torch.matmul for the base product alone (same shape,
    bf16; an FP8 base is widened to bf16 first): the vendor-library figure the
    fused kernel is compared with."""
    import torch

    w = inst.W0
    if w.dtype == torch.uint8:
        w = w.view(torch.float8_e4m3fn).to(torch.bfloat16)
    wt = w.t()
    out = torch.empty((inst.prob.T, inst.prob.d_out), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(5):
            torch.matmul(inst.x, wt, out=out)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch.matmul(inst.x, wt, out=out)
        e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def rotation_count(bytes_per_instance):
    n = max(8, math.ceil(2 * MALL_BYTES / max(bytes_per_instance, 1)))
    return 1 << (n - 1).bit_length()


HOST_CORES = 16  # the host CPU share of one GPU on the benchmark machine


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _prefix(prob, n):
    import copy

    sub = copy.copy(prob)
    sub.T = n
    sub.ids = prob.ids[:n]
    sub.x = prob.x[:n]
    sub.y_in = None if prob.y_in is None else prob.y_in[:n]
    return sub


def cpu_baseline(prob, budget_s):
    """The fp64 oracle as it stands, on the host cores (the machine's CPU share
    of one GPU, HOST_CORES threads, or fewer if fewer exist) and on one thread:
    median of 3 timed runs each, over whole layers of the same workload, or
    over a prefix of its tokens when a layer would not fit the budget."""
    import oracle

    fused = bool(prob.meta.get("fused"))
    cores = max(1, min(HOST_CORES, os.cpu_count() or 1))
    oracle.build(force=False)
    n_probe = min(prob.T, 8)
    t0 = time.perf_counter()
    oracle.lora_forward(_prefix(prob, n_probe), nthreads=1, fused=fused)
    per_tok_1 = (time.perf_counter() - t0) / n_probe

    def med_rate(sample, nthreads, reps=3):
        rates = []
        for _ in range(reps):
            t = time.perf_counter()
            oracle.lora_forward(sample, nthreads=nthreads, fused=fused)
            rates.append(sample.T / (time.perf_counter() - t))
        return float(np.median(rates)), rates

    # multi-thread leg: about 2/3 of the budget over 3 runs; whole layers when they fit
    per_run = budget_s * 2 / 9
    n_mt = prob.T if per_tok_1 * prob.T / cores <= per_run else max(cores, min(prob.T, int(per_run / per_tok_1 * cores)))
    mt, _ = med_rate(_prefix(prob, n_mt), cores)
    # one-thread leg: the rest of the budget
    per_run1 = budget_s / 9
    n_1 = max(1, min(prob.T, int(per_run1 / per_tok_1)))
    one, _ = med_rate(_prefix(prob, n_1), 1)
    what = "full layers" if n_mt == prob.T else f"the first {n_mt} of {prob.T} tokens of one layer"
    return {"value": mt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what}, median of 3 runs, fp64, OpenMP over tokens",
            "value_1thread": one, "sample_1thread": f"the first {n_1} tokens, median of 3 runs",
            "host_nproc": os.cpu_count(), "cpu_model": cpu_model()}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
KERNEL_SOURCES = {"fused": ["segmented_gather_gemm_lora_amd/csrc/fused.hip"]}
COPY_CAL_BYTES = 256 << 20


def kernel_source_digest(dominant):
    """sha256 over the source files that define the kernel, so that recorded
    counter figures are used only for the code they were taken on."""
    import hashlib

    files = KERNEL_SOURCES.get(dominant, ["segmented_gather_gemm_lora_amd/csrc/sgmv_bgmv.hip"])
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload, role):
    """HBM bytes per launch of the workload's `role` kernel (shrink, expand,
    fused) from the FETCH_SIZE and WRITE_SIZE counter runs recorded in
    profiles/hbm_traffic.md (each scaled by the factor the same counter gives
    for a copy of known size), with the kernel's name; (None, None) when no
    figures exist or the kernel source has changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            line = next(l for l in fh if l.startswith("traffic-json: "))
        rec = json.loads(line[len("traffic-json: "):])
    except (OSError, StopIteration, ValueError):
        return None, None
    e = rec.get("entries", {}).get(f"{workload}/{role}")
    if not e or e.get("source_sha256") != kernel_source_digest(role):
        return None, None
    return e.get("bytes_per_launch"), e.get("kernel")


def copy_calibration(reps=8):
    """Plain device-to-device copies of COPY_CAL_BYTES each: the known-size
    kernel that scales the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_CAL_BYTES, "reps": reps}))


def timed_steps(tm, steps, K, W, use_graph):
    """The contract's timed region: K steps after set-up, issued one library
    call at a time (or, with use_graph, replayed from a graph).  The other
    mode is timed beside it.  Returns (ms_per_step, wall_s, mode, other_ms,
    note)."""
    L = len(steps)
    eager_ms, eager_wall = tm.eager(steps, K, first=W % L)
    try:
        graph_ms, graph_wall = tm.graph(steps, K, first=W % L)
    except Exception as e:  # capture unsupported: report the eager figure
        return eager_ms, eager_wall, "eager", None, f"graph capture failed: {e}"
    if use_graph:
        return graph_ms, graph_wall, "graph", eager_ms, None
    return eager_ms, eager_wall, "eager", graph_ms, None


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", choices=sorted(CONFIG_OF) + ["decode_qkv", "prefill_qkv", "decode_cache"],
                    default="decode")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="report the K steps replayed from a graph (default: issued one call at a time)")
    ap.add_argument("--probe", action="store_true", help="only run the probes for the workload's bytes and exit")
    ap.add_argument("--rotation", type=int, default=None, help="override the number of rotated instances")
    ap.add_argument("--paged", type=int, default=0, metavar="PAGE_BYTES",
                    help="adapters in a page pool of this page size (decode, prefill, hetero); 0 = dense pool")
    ap.add_argument("--path", choices=["bgmv", "sgmv"], default=None,
                    help="run the decode workload through this call (default: bgmv)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain copies of a known size (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from lora_workloads import CONFIG_NAMES, FUSED_FP8_NAME, make_config, make_fused_fp8
    from segmented_gather_gemm_lora_amd import binding as B

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        copy_calibration()
        return
    B.load()
    stream = torch.cuda.Stream()  # default priority
    if args.config in ("decode_qkv", "prefill_qkv"):
        grouped_main(args, stream, sgmv=args.config == "prefill_qkv")
        return
    if args.config == "decode_cache":
        cache_main(args, stream)
        return
    k = CONFIG_OF[args.config]
    kind = {1: "sgmv", 2: "bgmv", 3: "sgmv", 4: "sgmv", 5: "fused"}[k]
    if args.path and k == 2:
        kind = args.path
    page = args.paged
    if page and kind == "fused":
        print("--paged applies to the SGMV/BGMV workloads, not the fused layer", file=sys.stderr)
        sys.exit(2)

    fp8 = args.config == "fused_fp8"
    wname = FUSED_FP8_NAME if fp8 else CONFIG_NAMES[k]

    def make(seed=None):
        if fp8:  # the fused workload over an FP8 (E4M3) base
            return make_fused_fp8(k if seed is None else seed)
        return make_config(k, seed=seed)

    prob0 = make()
    ab = algorithmic_bytes(prob0)
    L = args.rotation or rotation_count(ab["total"])
    print(f"[bench] {wname}: T={prob0.T} d_in={prob0.d_in} d_out={prob0.d_out} rotation={L} "
          f"bytes/layer={ab['total']/1e6:.2f} MB", file=sys.stderr, flush=True)
    if args.probe:
        rmw = 0 if kind == "fused" else int(np.count_nonzero(prob0.ids >= 0)) * prob0.d_out * prob0.esize
        print(json.dumps({"workload": wname, "probes": run_probes(stream, ab["total"] - 2 * rmw, rmw, L)}))
        return
    insts = [Instance(prob0, kind, stream, page, seed=0)]
    for i in range(1, L):
        insts.append(Instance(make(1000 * k + i), kind, stream, page, seed=i))
    torch.cuda.synchronize()
    # every instance has its own distinct-adapter count; average the algorithmic bytes
    ab_all = [algorithmic_bytes(inst.prob) for inst in insts]
    bytes_step = float(np.mean([a["total"] for a in ab_all]))
    flops_step = float(np.mean([algorithmic_flops(inst.prob) for inst in insts]))
    T = prob0.T
    steps = [inst.step for inst in insts]

    K = args.steps if args.steps is not None else 20 * L
    W = args.warmup if args.warmup is not None else 10 * L
    tm = Timing(stream)
    tm.setup(steps, W)
    used = launches_per_step(steps[0])
    if kind == "fused":
        names = ["shrink", "prep", "fused"]
    elif used == 1:
        names = [kind]  # shrink and expand in one kernel
    else:
        names = ["shrink", "expand"]
    assert len(names) == used, (names, used)

    # ---- timed region: exactly K steps
    ms_step, t_wall, mode, other_ms, graph_note = timed_steps(tm, steps, K, W, args.graph)
    tokens_per_s = T / (ms_step * 1e-3)
    gbps = bytes_step / (ms_step * 1e-3) / 1e9

    # ---- per-kernel durations: HIP events attached to each kernel's own start
    # and end (hipExtLaunchKernelGGL), on the stream the kernels run on
    K2 = max(L, min(K, 20 * L))
    per_kernel_us = tm.per_kernel(steps, names, K2)
    dominant = max(names, key=lambda n: per_kernel_us[n])
    dom_us = per_kernel_us[dominant]
    if kind != "fused" and names == [kind]:
        for a in ab_all:
            a[kind] = a["total"]
    dom_bytes = float(np.mean([a.get(dominant, a["total"]) for a in ab_all]))
    if kind == "fused":
        dominant = "fused"
        dom_us = per_kernel_us["fused"]
        dom_bytes = float(np.mean([a["fused"] for a in ab_all]))
        fused_flops = float(np.mean([algorithmic_flops(inst.prob, "fused") for inst in insts]))
        achieved = fused_flops / (dom_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}
    traffic, kname = recorded_traffic(wname + (f"_paged{page}" if page else ""), dominant)
    roof["traffic"] = traffic
    default_names = {"shrink": f"{kind}_shrink", "expand": f"{kind}_expand", "fused": "fused_linear"}
    if names == [kind]:
        default_names[kind] = f"{kind}_onepass"
    roof["kernel"] = kname or default_names[dominant]
    roof["algorithmic_bytes_per_launch"] = round(dom_bytes)
    roof["avg_launch_us"] = round(dom_us, 3)

    extra = {}
    if kind == "fused":
        roof["algorithmic_flops_per_launch"] = round(fused_flops)
        base_us = base_gemm_reference_us(insts[0], stream)
        extra = {"base_gemm_reference_us": round(base_us, 3), "base_gemm_reference": "torch.matmul (hipBLASLt), "
                 "x [T, d_in] @ W0^T, bf16, same shape, no adapters; a library reference, not part of the path"}
    probes = None
    if not args.no_probes:
        # y of the adapted tokens is read and written back; everything else is read
        rmw = int(np.mean([np.count_nonzero(inst.prob.ids >= 0) * inst.prob.d_out * inst.prob.esize
                           for inst in insts])) if kind != "fused" else 0
        del insts, steps
        torch.cuda.empty_cache()
        probes = run_probes(stream, bytes_step - 2 * rmw, rmw, L)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(prob0, args.cpu_budget)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob0.dtype,
        "data": "synthetic",
        "config": {"workload": wname, "T": T, "d_in": prob0.d_in, "d_out": prob0.d_out,
                   "ranks": sorted(set(int(r) for r in prob0.ranks)), "pool_adapters": prob0.n_adapters,
                   "distinct_adapters": int(len(prob0.distinct_adapters())), "rotated_instances": L,
                   "path": kind + ("_paged" if page else ""), **({"page_bytes": page} if page else {}),
                   **({"w0_format": "e4m3", "w0_scale": "one fp32 per matrix"} if fp8 else {})},
        "timed_mode": mode,
        ("graph_ms_per_step" if mode == "eager" else "eager_ms_per_step"):
            None if other_ms is None else round(other_ms, 6),
        "achieved_GBps": round(gbps, 1),
        "hbm_peak_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": round(bytes_step),
        "algorithmic_flops_per_step": round(flops_step),
        "per_kernel_us": {n: round(v, 3) for n, v in per_kernel_us.items()},
        "kernel_sum_us": round(sum(per_kernel_us.values()), 3),
        "probes": probes,
        "wall_s_timed": round(t_wall, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if graph_note:
        out["graph_note"] = graph_note
    out.update(extra)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
