#!/usr/bin/env python3
"""Benchmark of the sparse-attention hot path on one MI355X.

Headline: 1M-context decode attention, one step = hierarchical pruning (three
stages) + sparse attention for one new query of a batch-1 sequence with 32
query / 8 KV heads, d=128, T=1,048,576 bf16, through dsa_prune_attend (the
one-call step; the two-call prune_select + sparse_attn figure is reported
next to it). Reported as microseconds per token, with the step's algorithmic
HBM bytes / time against the 8 TB/s HBM peak.

Secondary figures on the same JSON line: 128K sparse prefill TFLOP/s against
the bf16 MFMA peak, the library's dense decode at 1M, per-kernel durations
from HIP events on the launch stream, and the CPU oracle timed on the host.

    python bench.py [--steps K] [--warmup W] [--no-prefill] [--no-dense] [--no-cached] [--no-cpu]

Also on the line: decoding with remembered stage outputs (mask caching, the
default refresh intervals 16/8/4) at 1M, as amortised microseconds per token.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn us/token @1M ctx (HBM GB/s, % peak); 128K sparse prefill TFLOP/s"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _counter_summary(name: str):
    """Machine-readable fields of a committed rocprofv3 counter summary under
    profiles/, or None if it is missing or its kernel sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if ":" in line and not line.startswith(("|", "#", "rocprofv3")):
            key, val = line.split(":", 1)
            if key.isidentifier():
                kv[key] = val.strip()
    if "source_files" not in kv:
        return None
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in kv["source_files"].split()))
    if h.hexdigest() != kv.get("source_sha256"):
        return None
    return kv


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if there is none or the kernel source changed since."""
    kv = _counter_summary("decode_1m_counters.md")
    if not kv or kv.get("traffic_kernel") != kernel:
        return None
    return int(kv["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=8,
                    help="KV copies cycled through so consecutive steps share no cache lines")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--graph-steps", type=int, default=8,
                    help="decode steps captured per HIP graph (a model captures a whole decode step)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cached", action="store_true", help="skip decoding with remembered stages")
    ap.add_argument("--no-other", action="store_true", help="skip the batch-32 paged and 3M-token decodes")
    ap.add_argument("--no-block-sparse", action="store_true", help="skip the block-sparse heads prefill")
    ap.add_argument("--no-vertical-slash", action="store_true", help="skip the vertical-slash heads prefill")
    ap.add_argument("--no-rope", action="store_true", help="skip pruning with RoPE in SelectRep (both styles)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


# --------------------------------------------------------------------------- #
# per-kernel durations in graph mode                                          #
# --------------------------------------------------------------------------- #
class _Dim3(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint32), ("y", ctypes.c_uint32), ("z", ctypes.c_uint32)]


class _KernelNodeParams(ctypes.Structure):
    _fields_ = [("blockDim", _Dim3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p),
                ("gridDim", _Dim3), ("kernelParams", ctypes.c_void_p), ("sharedMemBytes", ctypes.c_uint32)]


def graph_kernel_times(launches, repeat=16, reps=4):
    """Average duration (us) of each kernel of one step, in launch order.

    Eager launches on this GPU pay a large per-launch release between dependent
    kernels, so kernels are timed in graph mode instead: each callable in
    `launches` (the same step on different KV replicas) is captured into a HIP
    graph; for each kernel position a graph chaining `repeat` copies of that
    kernel node, cycling through the captures so consecutive copies read
    different replicas (no cache reuse), is replayed `reps` times between HIP
    events on the launch stream. Every library kernel is idempotent given the
    step's final state, so re-running a node reproduces its real work."""
    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    vp = ctypes.c_void_p

    def ck(err, what):
        if err != 0:
            raise RuntimeError(f"{what} failed with HIP error {err}")

    stream = torch.cuda.Stream()
    graphs, chains = [], []
    for launch in launches:
        graph = vp()
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            ck(hip.hipStreamBeginCapture(vp(stream.cuda_stream), 0), "hipStreamBeginCapture")
            launch()
            ck(hip.hipStreamEndCapture(vp(stream.cuda_stream), ctypes.byref(graph)), "hipStreamEndCapture")
        graphs.append(graph)
        # walk the captured chain from its root
        nodes = []
        n = ctypes.c_size_t(1)
        root = vp()
        ck(hip.hipGraphGetRootNodes(graph, ctypes.byref(root), ctypes.byref(n)), "hipGraphGetRootNodes")
        node = root if n.value == 1 else None
        while node is not None and node.value:
            ty = ctypes.c_int(-1)
            ck(hip.hipGraphNodeGetType(node, ctypes.byref(ty)), "hipGraphNodeGetType")
            if ty.value == 0:
                prm = _KernelNodeParams()
                ck(hip.hipGraphKernelNodeGetParams(node, ctypes.byref(prm)), "hipGraphKernelNodeGetParams")
                nodes.append(prm)
            nd = ctypes.c_size_t(1)
            nxt = vp()
            ck(hip.hipGraphNodeGetDependentNodes(node, ctypes.byref(nxt), ctypes.byref(nd)),
               "hipGraphNodeGetDependentNodes")
            node = nxt if nd.value == 1 else None
        chains.append(nodes)
    times = []
    for k in range(len(chains[0])):
        g2 = vp()
        ck(hip.hipGraphCreate(ctypes.byref(g2), ctypes.c_uint(0)), "hipGraphCreate")
        prev = vp()
        for i in range(repeat):
            prm = chains[i % len(chains)][k]
            cur = vp()
            deps = ctypes.byref(prev) if i else None
            ck(hip.hipGraphAddKernelNode(ctypes.byref(cur), g2, deps, ctypes.c_size_t(1 if i else 0),
                                         ctypes.byref(prm)), "hipGraphAddKernelNode")
            prev = cur
        ex = vp()
        ck(hip.hipGraphInstantiate(ctypes.byref(ex), g2, None, None, ctypes.c_size_t(0)), "hipGraphInstantiate")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ck(hip.hipGraphLaunch(ex, vp(stream.cuda_stream)), "hipGraphLaunch")     # warm
        e0.record(stream)
        for _ in range(reps):
            ck(hip.hipGraphLaunch(ex, vp(stream.cuda_stream)), "hipGraphLaunch")
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / (reps * repeat))
        hip.hipGraphExecDestroy(ex)
        hip.hipGraphDestroy(g2)
    for g in graphs:
        hip.hipGraphDestroy(g)
    return times


# --------------------------------------------------------------------------- #
# decode at 1M                                                                #
# --------------------------------------------------------------------------- #
def decode_bench(args, res):
    import torch
    from dynamic_sparse_attention_query_amd import _lib, gen
    from dynamic_sparse_attention_query_amd._lib import DSA_BF16, DSA_DECODE, Shape
    from dynamic_sparse_attention_query_amd.inputs import params_of, to_device

    t0 = time.time()
    case = gen.make_case("c3")
    cfg = case.cfg
    dev = to_device(case)
    log(f"decode inputs ready in {time.time() - t0:.1f}s")
    p = params_of(cfg)
    lib = _lib.load()
    T, Hq, Hkv, d = cfg.t, cfg.hq, cfg.hkv, cfg.d
    Ks = [dev.k] + [dev.k.clone() for _ in range(args.replicas - 1)]
    Vs = [dev.v] + [dev.v.clone() for _ in range(args.replicas - 1)]
    NQ = dev.q.shape[0]
    Qs = [dev.q[i].contiguous() for i in range(NQ)]
    shape = Shape(DSA_DECODE, DSA_BF16, 1, Hq, Hkv, d, T, seq_lens=dev.seq_lens.data_ptr())
    L = _lib.index_width(p)
    wsb = _lib.workspace_bytes(shape, p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    idx = torch.empty(L, dtype=torch.int32, device="cuda")
    out = torch.empty((1, Hq, d), dtype=torch.float32, device="cuda")
    cs, cp = shape.c(), p.c()

    def launch_two(i, visited=None):
        q, r = Qs[i % NQ], i % args.replicas
        sp = torch.cuda.current_stream().cuda_stream
        st = lib.dsa_prune_select(ctypes.byref(cs), q.data_ptr(), Ks[r].data_ptr(), ctypes.byref(cp),
                                  idx.data_ptr(), ws.data_ptr(), wsb,
                                  visited.data_ptr() if visited is not None else None, sp)
        st |= lib.dsa_sparse_attn(ctypes.byref(cs), q.data_ptr(), Ks[r].data_ptr(), Vs[r].data_ptr(),
                                  idx.data_ptr(), L, 1, 0.0, out.data_ptr(), ws.data_ptr(), wsb, sp)
        if st:
            raise RuntimeError(lib.dsa_last_error().decode())

    def launch(i, visited=None):
        q, r = Qs[i % NQ], i % args.replicas
        sp = torch.cuda.current_stream().cuda_stream
        st = lib.dsa_prune_attend(ctypes.byref(cs), q.data_ptr(), Ks[r].data_ptr(), Vs[r].data_ptr(),
                                  ctypes.byref(cp), 0.0, idx.data_ptr(), out.data_ptr(), ws.data_ptr(), wsb,
                                  visited.data_ptr() if visited is not None else None, sp)
        if st:
            raise RuntimeError(lib.dsa_last_error().decode())

    # algorithmic bytes of each query's step: distinct K rows SelectRep reads
    # (counted by the kernels) + K and V rows of every kept key
    row_bytes = d * 2
    stage_bytes = np.zeros((NQ, len(p.chunk)))
    attn_bytes = np.zeros(NQ)
    vis = torch.zeros(len(p.chunk), dtype=torch.int64, device="cuda")
    for i in range(NQ):
        vis.zero_()
        launch(i, vis)
        torch.cuda.synchronize()
        stage_bytes[i] = vis.cpu().numpy() * row_bytes
        attn_bytes[i] = int((idx >= 0).sum().item()) * Hkv * 2 * row_bytes
    step_bytes = stage_bytes.sum(1) + attn_bytes

    K, W = args.steps, args.warmup
    GS = args.graph_steps if args.graph_steps > 0 and K % args.graph_steps == 0 else 1

    def timed(fn):
        """(wall us/step, event us/step, wall ms, step indices) of K steps after
        the warm-up: graph replays of GS steps each (step i uses query i mod NQ
        and KV replica i mod replicas), or eager launches with --eager."""
        n_w = max(1, W // GS)
        n_runs = K // GS if not args.eager else K
        steps_of = lambda j: list(range(j * GS, j * GS + GS)) if not args.eager else [j]
        graphs = None
        if not args.eager:
            graphs = []
            torch.cuda.synchronize()
            for j in range(n_w + n_runs):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in steps_of(j):
                        fn(i)
                graphs.append(g)
            torch.cuda.synchronize()

        def run(j):
            if graphs is not None:
                graphs[j].replay()
            else:
                fn(j)

        for j in range(n_w):
            run(j)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_start = time.perf_counter()
        e0.record()
        for j in range(n_w, n_w + n_runs):
            run(j)
        e1.record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t_start) * 1e3
        del graphs
        steps = [i for j in range(n_w, n_w + n_runs) for i in steps_of(j)]
        return wall_ms * 1e3 / K, e0.elapsed_time(e1) * 1e3 / K, wall_ms, steps

    us_step, ev_us, wall_ms, steps = timed(launch)
    two_us, _, _, _ = timed(launch_two)
    used = [i % NQ for i in steps]
    bytes_avg = float(step_bytes[used].mean())
    log(f"decode 1M: {us_step:.1f} us/step wall, {ev_us:.1f} us/step events ({GS} steps per graph); "
        f"two-call path {two_us:.1f} us/step")

    # per-kernel durations: HIP events around graph replays of each kernel of a
    # captured step (kernel names from the library's own launch record)
    _lib.profile_begin()
    launch(W)
    prof = _lib.profile_end()
    names = list(prof.keys())
    gt = graph_kernel_times([lambda i=i: launch(i) for i in range(W, W + args.replicas)])
    if len(gt) != len(names):
        raise RuntimeError(f"captured {len(gt)} kernels, expected {len(names)}")
    kern_us = dict(zip(names, gt))
    per_launch_bytes = {
        "prune_score_stage1": float(stage_bytes[used, 0].mean()),
        "prune_topk1_score2": float(stage_bytes[used, 1].mean()),
        "prune_topk2_score3": float(stage_bytes[used, 2].mean()),
        "decode_topk_attend_partial": float(attn_bytes[used].mean()),
    }
    dom = max(kern_us, key=kern_us.get)
    roof = None
    if dom in per_launch_bytes:
        ach = per_launch_bytes[dom] / (kern_us[dom] * 1e-6) / 1e9
        tr = measured_traffic(dom)
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": tr,
                "avg_us": round(kern_us[dom], 2), "algorithmic_bytes_per_launch": int(per_launch_bytes[dom])}
    # per-step distribution: each of 64 steps (fresh query, KV replica cycled)
    # replayed alone between HIP events, cache-cold (a 1 GiB read before it,
    # outside the timed region) and without the flush
    n_ps = 64
    one = []
    for i in range(min(n_ps, NQ * args.replicas)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch(i)
        one.append(g)
    for g in one:
        g.replay()
    torch.cuda.synchronize()
    junk = torch.zeros((1 << 30) // 4, dtype=torch.float32, device="cuda")
    flush = torch.zeros((), dtype=torch.float32, device="cuda")
    torch.sum(junk, dim=0, out=flush)
    per_step = {}
    for mode in ("cold", "warm"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ps)]
        for i in range(n_ps):
            if mode == "cold":
                torch.sum(junk, dim=0, out=flush)      # read: the caches end clean
            evs[i][0].record()
            one[i % len(one)].replay()
            evs[i][1].record()
            if mode == "warm":
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t = np.array([a_.elapsed_time(b_) * 1e3 for a_, b_ in evs])
        per_step[mode] = (float(np.median(t)), float(np.percentile(t, 90)), float(t.mean()))
    del one, junk, flush
    log(f"decode 1M per step: cache-cold median {per_step['cold'][0]:.1f} us, p90 {per_step['cold'][1]:.1f}; "
        f"without the flush median {per_step['warm'][0]:.1f}, p90 {per_step['warm'][1]:.1f}")

    res["decode"] = dict(us_per_step=us_step, event_us_per_step=ev_us, wall_ms=wall_ms, per_step=per_step,
                         two_call_us_per_step=two_us, graph_steps=GS,
                         bytes_per_step=bytes_avg, stage_rows=(stage_bytes[used].mean(0) / row_bytes).tolist(),
                         kernels_us={k: round(v, 2) for k, v in kern_us.items()}, roofline=roof,
                         mode="graph" if not args.eager else "eager")

    if not args.no_cached:
        res["cached"] = cached_decode(args, lib, p, Qs, Ks, Vs, shape, ws, wsb, out, dev.seq_lens)

    if not args.no_dense:
        reps = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dshape_ws = _lib.workspace_bytes(shape, None)
        dws = torch.empty(dshape_ws, dtype=torch.uint8, device="cuda")
        for i in range(reps + 1):
            if i == 1:
                torch.cuda.synchronize()
                e0.record()
            r = i % args.replicas
            st = lib.dsa_dense_attn(ctypes.byref(cs), Qs[i].data_ptr(), Ks[r].data_ptr(), Vs[r].data_ptr(),
                                    0.0, out.data_ptr(), dws.data_ptr(), dshape_ws,
                                    torch.cuda.current_stream().cuda_stream)
            if st:
                raise RuntimeError(lib.dsa_last_error().decode())
        e1.record()
        torch.cuda.synchronize()
        dense_us = e0.elapsed_time(e1) * 1e3 / reps
        kv_bytes = 2 * Hkv * T * d * 2
        res["dense"] = dict(us=dense_us, gbps=kv_bytes / (dense_us * 1e-6) / 1e9, bytes=kv_bytes)
        del dws
    del Ks, Vs, dev, ws
    torch.cuda.empty_cache()
    return case


def cached_decode(args, lib, p, Qs, Ks, Vs, shape, ws, wsb, out, seq_lens_full, refresh=(16, 8, 4)):
    """Decode with remembered stage outputs at 1M: one refresh cycle of
    refresh[0] steps (every stage due at step 0, then each stage at its own
    interval), the context growing by one token per step up to T, a fresh query
    and the next KV replica each step. Returns the amortised time per token."""
    import torch
    from dynamic_sparse_attention_query_amd import _lib
    from dynamic_sparse_attention_query_amd._lib import Shape
    n = refresh[0]
    T = shape.t
    NQ = len(Qs)
    sls = [torch.full((1,), T - n + 1 + i, dtype=torch.int32, device="cuda") for i in range(n)]
    shapes = [Shape(shape.mode, shape.dtype, 1, shape.hq, shape.hkv, shape.d, T, seq_lens=sl.data_ptr())
              for sl in sls]
    cshapes = [sh.c() for sh in shapes]
    cp = p.c()
    L = _lib.cached_index_width(p, n - 1)
    cb = _lib.mask_cache_bytes(shapes[0], p)
    cache = torch.zeros(cb, dtype=torch.uint8, device="cuda")
    idx = torch.empty(L, dtype=torch.int32, device="cuda")
    rf = (ctypes.c_int32 * 4)(*(list(refresh) + [1] * (4 - len(refresh))))

    def launch(i, visited=None):
        step = i % n
        q, r = Qs[i % NQ], i % args.replicas
        sp = torch.cuda.current_stream().cuda_stream
        cs = cshapes[step]
        st = lib.dsa_prune_select_cached(ctypes.byref(cs), q.data_ptr(), Ks[r].data_ptr(), ctypes.byref(cp),
                                         rf, step, cache.data_ptr(), cb, idx.data_ptr(), L, ws.data_ptr(), wsb,
                                         visited.data_ptr() if visited is not None else None, sp)
        st |= lib.dsa_sparse_attn(ctypes.byref(cs), q.data_ptr(), Ks[r].data_ptr(), Vs[r].data_ptr(),
                                  idx.data_ptr(), L, 1, 0.0, out.data_ptr(), ws.data_ptr(), wsb, sp)
        if st:
            raise RuntimeError(lib.dsa_last_error().decode())

    # algorithmic bytes of one cycle: SelectRep rows of the stages that ran
    # (counted by the kernels) + K and V rows of every step's kept keys
    row_bytes = shape.d * 2
    vis = torch.zeros(len(p.chunk), dtype=torch.int64, device="cuda")
    cyc_bytes = 0.0
    for i in range(n):
        launch(i, vis)
        torch.cuda.synchronize()
        cyc_bytes += int((idx >= 0).sum().item()) * shape.hkv * 2 * row_bytes
    cyc_bytes += float(vis.sum().item()) * row_bytes
    assert int(cache[:4].view(torch.int32).item()) == 0, "cached row overflow"

    graphs = []
    torch.cuda.synchronize()
    for i in range(n * 2):                       # two cycles: replicas alternate between them
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch(i)
        graphs.append(g)
    torch.cuda.synchronize()
    cycles = max(2, args.steps // n)
    for i in range(n * 2):
        graphs[i].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for c in range(cycles):
        for i in range(n):
            graphs[(c % 2) * n + i].replay()
    e1.record()
    torch.cuda.synchronize()
    us_tok = e0.elapsed_time(e1) * 1e3 / (cycles * n)
    # per-step-kind times: a step with every stage due vs one that only assembles
    def step_us(i, reps=8):
        e0.record()
        for _ in range(reps):
            graphs[i].replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps
    full_us, reuse_us = step_us(0), step_us(1)
    log(f"cached decode 1M {refresh}: {us_tok:.1f} us/token amortised "
        f"(all stages due {full_us:.1f} us, none due {reuse_us:.1f} us)")
    return dict(refresh=list(refresh), us_per_token=us_tok, steps=cycles * n,
                bytes_per_token=cyc_bytes / n, full_refresh_step_us=full_us, reuse_step_us=reuse_us)


# --------------------------------------------------------------------------- #
# prefill at 128K                                                             #
# --------------------------------------------------------------------------- #
def prefill_block_flops(cfg):
    """Per query block: algorithmic flops of the SelectRep evaluations and of
    the attention, from the geometry alone (the row of block m holds the
    sinks, the kept keys of the last stage and the window up to the block's
    end)."""
    bq, d, Hq = cfg.block_q, cfg.d, cfg.hq
    nblk = cfg.t // bq
    sel = np.zeros(nblk)
    attn = np.zeros(nblk)
    for m in range(nblk):
        e = (m + 1) * bq
        n1 = max(0, e - cfg.n_window - cfg.n_sink) // cfg.chunk[0]
        nc = n1
        for i, (l, k) in enumerate(zip(cfg.chunk, cfg.keep)):
            if i > 0:
                nc = kept * (cfg.chunk[i - 1] // l)
            kc = k // l
            if nc > kc:
                sel[m] += nc * Hq * (1 + int(math.log2(l))) * bq * 2 * d
            kept = min(nc, kc)
        mid_hi = cfg.n_sink + n1 * cfg.chunk[0]
        n_row = min(cfg.n_sink, e) + kept * cfg.chunk[-1] + (e - mid_hi)
        attn[m] = (bq * (n_row - bq) + bq * (bq + 1) // 2) * Hq * 4 * d
    return sel, attn


def prefill_algorithmic_flops(cfg, n_row: np.ndarray):
    """SelectRep evaluations (b_q * 2d flops each, one per distinct representative
    per (chunk, query head) of every stage that prunes) and attention over the
    visible (query, key) pairs (4d flops each: q.k and p.v)."""
    bq, d, Hq = cfg.block_q, cfg.d, cfg.hq
    nblk = cfg.t // bq
    sel = 0
    for m in range(nblk):
        e = (m + 1) * bq
        nc = max(0, e - cfg.n_window - cfg.n_sink) // cfg.chunk[0]
        for i, (l, k) in enumerate(zip(cfg.chunk, cfg.keep)):
            if i > 0:
                nc = kept * (cfg.chunk[i - 1] // l)
            kc = k // l
            if nc > kc:
                sel += nc * Hq * (1 + int(math.log2(l)))
            kept = min(nc, kc)
    sel_flops = sel * bq * 2 * d
    assert cfg.n_window >= bq
    pairs = (bq * (n_row.astype(np.int64) - bq) + bq * (bq + 1) // 2).sum()
    attn_flops = int(pairs) * Hq * 4 * d
    return sel_flops, attn_flops


def prefill_bench(args, res):
    import torch
    from dynamic_sparse_attention_query_amd import _lib, api, gen
    from dynamic_sparse_attention_query_amd.inputs import params_of, to_device

    t0 = time.time()
    case = gen.make_case("c2_128k")
    cfg = case.cfg
    dev = to_device(case)
    del case
    log(f"prefill inputs ready in {time.time() - t0:.1f}s")
    p = params_of(cfg)
    idx = api.prune_select(dev.q, dev.k, p)
    out = api.sparse_attn(dev.q, dev.k, dev.v, idx, p)
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        api.prune_select(dev.q, dev.k, p, out=idx.view(-1))
        api.sparse_attn(dev.q, dev.k, dev.v, idx, p, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    _lib.profile_begin()
    api.prune_select(dev.q, dev.k, p, out=idx.view(-1))
    api.sparse_attn(dev.q, dev.k, dev.v, idx, p, out=out)
    prof = _lib.profile_end()
    n_row = (idx >= 0).sum(-1).view(-1).cpu().numpy()
    sel_f, attn_f = prefill_algorithmic_flops(cfg, n_row)
    tot = sel_f + attn_f
    prune_ms = sum(v[1] for k, v in prof.items() if k.startswith("prune_"))
    attn_ms = sum(v[1] for k, v in prof.items() if k.startswith("attn_"))
    res["prefill"] = dict(ms=ms, tflops=tot / (ms * 1e-3) / 1e12, algorithmic_tflop=tot / 1e12,
                          selectrep_tflop=sel_f / 1e12, attn_tflop=attn_f / 1e12,
                          prune_ms=prune_ms, attn_ms=attn_ms,
                          attn_tflops=attn_f / (attn_ms * 1e-3) / 1e12 if attn_ms else None,
                          kernels_ms={k: round(v[1] / v[0], 3) for k, v in prof.items()})
    log(f"prefill 128K: {ms:.1f} ms, {res['prefill']['tflops']:.1f} TFLOP/s")
    if not args.no_rope:
        res["rope_prefill"] = {}
        for style in ROPE_STYLES:
            idx_rt = api.prune_select_rope(dev.q, dev.k, p, ROPE_BASE, style=style)
            api.sparse_attn(dev.q, dev.k, dev.v, idx_rt, p, out=out)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                api.prune_select_rope(dev.q, dev.k, p, ROPE_BASE, out=idx_rt.view(-1), style=style)
                api.sparse_attn(dev.q, dev.k, dev.v, idx_rt, p, out=out)
            e1.record()
            torch.cuda.synchronize()
            ms_rt = e0.elapsed_time(e1) / reps
            _lib.profile_begin()
            api.prune_select_rope(dev.q, dev.k, p, ROPE_BASE, out=idx_rt.view(-1), style=style)
            prof_rt = _lib.profile_end()
            res["rope_prefill"][style] = dict(
                ms=ms_rt, prune_ms=sum(v[1] for v in prof_rt.values()), plain_ms=ms, plain_prune_ms=prune_ms,
                rows_changed=float((idx_rt != idx).any(-1).float().mean().item()),
                kernels_ms={k: round(v[1] / v[0], 3) for k, v in prof_rt.items()})
            log(f"prefill 128K with {style} RoPE: {ms_rt:.1f} ms "
                f"(pruning {res['rope_prefill'][style]['prune_ms']:.1f} ms)")
            del idx_rt
    del dev, idx, out
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- #
# block-sparse heads at the 128K prefill shape                                #
# --------------------------------------------------------------------------- #
BS_K_BLOCKS = 100          # the page's k_b for Block-Sparse heads


def block_sparse_bench(args, res, reps=3):
    """Block-sparse estimation + per-head attention over the 128K Llama-shaped
    prefill (k_b = 100), with the dense causal path at the same shape."""
    import torch
    from dynamic_sparse_attention_query_amd import _lib, api, gen
    from dynamic_sparse_attention_query_amd.inputs import to_device

    case = gen.make_case("c2_128k")
    cfg = case.cfg
    dev = to_device(case)
    del case
    idx = api.block_sparse_select(dev.q, dev.k, BS_K_BLOCKS)
    out = api.sparse_attn_heads(dev.q, dev.k, dev.v, idx)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        api.block_sparse_select(dev.q, dev.k, BS_K_BLOCKS, out=idx.view(-1))
        api.sparse_attn_heads(dev.q, dev.k, dev.v, idx, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    _lib.profile_begin()
    api.block_sparse_select(dev.q, dev.k, BS_K_BLOCKS, out=idx.view(-1))
    api.sparse_attn_heads(dev.q, dev.k, dev.v, idx, out=out)
    prof = _lib.profile_end()
    # visible (query, key) pairs: whole 64 x 64 blocks below the diagonal, the
    # causal half (64 * 65 / 2) of a kept diagonal block
    nblk, d, Hq = cfg.t // 64, cfg.d, cfg.hq
    starts = idx[..., ::64]
    m_pos = (torch.arange(nblk, device=idx.device, dtype=torch.int32) * 64).view(1, 1, nblk, 1)
    below = ((starts >= 0) & (starts < m_pos)).sum().item()
    diag = (starts == m_pos).sum().item()
    pairs = below * 64 * 64 + diag * (64 * 65 // 2)
    attn_f = pairs * 4 * d
    est_f = Hq * cfg.batch * (nblk * (nblk + 1) // 2) * 2 * d          # pooled logits (fp64)
    est_ms = sum(v[1] for k, v in prof.items() if k.startswith("bs_"))
    attn_ms = sum(v[1] for k, v in prof.items() if k.startswith("attn_"))
    dense_ms = None
    if not args.no_dense:
        api.dense_attn(dev.q, dev.k, dev.v, out=out)
        torch.cuda.synchronize()
        e0.record()
        api.dense_attn(dev.q, dev.k, dev.v, out=out)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1)
    res["block_sparse"] = dict(ms=ms, attn_tflop=attn_f / 1e12, est_tflop_fp64=est_f / 1e12,
                               est_ms=est_ms, attn_ms=attn_ms, dense_ms=dense_ms,
                               kernels_ms={k: round(v[1] / v[0], 3) for k, v in prof.items()},
                               row_index_bytes=idx.numel() * 4)
    log(f"block-sparse 128K: {ms:.2f} ms (estimation {est_ms:.2f}, attention {attn_ms:.2f}), "
        f"{attn_f / (ms * 1e-3) / 1e12:.1f} TFLOP/s" + (f", dense {dense_ms:.1f} ms" if dense_ms else ""))
    # the same selection as block lists (the page's kernel takes block ids)
    # and the attention over them
    blocks, counts = api.block_sparse_select_lists(dev.q, dev.k, BS_K_BLOCKS)
    api.sparse_attn_lists(dev.q, dev.k, dev.v, blocks, counts, out=out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        api.block_sparse_select_lists(dev.q, dev.k, BS_K_BLOCKS, blocks=blocks, counts=counts)
        api.sparse_attn_lists(dev.q, dev.k, dev.v, blocks, counts, out=out)
    e1.record()
    torch.cuda.synchronize()
    lms = e0.elapsed_time(e1) / reps
    _lib.profile_begin()
    api.block_sparse_select_lists(dev.q, dev.k, BS_K_BLOCKS, blocks=blocks, counts=counts)
    api.sparse_attn_lists(dev.q, dev.k, dev.v, blocks, counts, out=out)
    lprof = _lib.profile_end()
    res["block_sparse"]["lists"] = dict(
        ms=lms, est_ms=sum(v[1] for k, v in lprof.items() if k.startswith("bs_")),
        attn_ms=sum(v[1] for k, v in lprof.items() if k.startswith("attn_")),
        index_bytes=(blocks.numel() + counts.numel()) * 4)
    log(f"block-sparse 128K, block lists: {lms:.2f} ms")
    del dev, idx, out, blocks, counts
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- #
# vertical-slash heads at the 128K prefill shape                              #
# --------------------------------------------------------------------------- #
VS_KEEP = (3000, 200)      # (k_v, k_s), one of the page's searched settings


def visible_pairs(idx, chunk_heads=4):
    """(query, key) pairs the rows [B, Hq, nblk, L] admit under the causal
    mask: 64 per entry before the block, e - p for an entry p inside it."""
    import torch
    nblk = idx.shape[2]
    s = (torch.arange(nblk, device=idx.device, dtype=torch.int64) * 64).view(1, 1, nblk, 1)
    total = 0
    for h0 in range(0, idx.shape[1], chunk_heads):
        x = idx[:, h0:h0 + chunk_heads].to(torch.int64)
        before = ((x >= 0) & (x < s)).sum().item()
        inside = torch.where((x >= s) & (x < s + 64), s + 64 - x, torch.zeros_like(x)).sum().item()
        total += 64 * before + inside
        del x
    return total


def vertical_slash_bench(args, res, reps=3):
    import torch
    from dynamic_sparse_attention_query_amd import _lib, api, gen
    from dynamic_sparse_attention_query_amd.inputs import to_device

    case = gen.make_case("c2_128k", structure="local", n_needles=0)
    cfg = case.cfg
    dev = to_device(case)
    del case
    k_v, k_s = VS_KEEP
    idx = api.vertical_slash_select(dev.q, dev.k, k_v, k_s)
    out = api.sparse_attn_heads(dev.q, dev.k, dev.v, idx)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        api.vertical_slash_select(dev.q, dev.k, k_v, k_s, out=idx.view(-1))
        api.sparse_attn_heads(dev.q, dev.k, dev.v, idx, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    _lib.profile_begin()
    api.vertical_slash_select(dev.q, dev.k, k_v, k_s, out=idx.view(-1))
    api.sparse_attn_heads(dev.q, dev.k, dev.v, idx, out=out)
    prof = _lib.profile_end()
    pairs = visible_pairs(idx)
    entries = (idx >= 0).sum().item() / (idx.shape[0] * idx.shape[1] * idx.shape[2])
    attn_f = pairs * 4 * cfg.d
    est_ms = sum(v[1] for k, v in prof.items() if k.startswith("vs_"))
    attn_ms = sum(v[1] for k, v in prof.items() if k.startswith("attn_"))
    res["vertical_slash"] = dict(ms=ms, attn_tflop=attn_f / 1e12, est_ms=est_ms, attn_ms=attn_ms,
                                 entries=entries, width=idx.shape[-1],
                                 kernels_ms={k: round(v[1] / v[0], 3) for k, v in prof.items()},
                                 row_index_bytes=idx.numel() * 4)
    log(f"vertical-slash 128K {VS_KEEP}: {ms:.2f} ms (estimation {est_ms:.2f}, attention {attn_ms:.2f}), "
        f"{attn_f / (ms * 1e-3) / 1e12:.1f} TFLOP/s, {entries:.0f} keys per row")
    # the hybrid kernel's form: block and column lists, blocks loaded as
    # contiguous tiles, columns gathered
    del idx
    torch.cuda.empty_cache()
    blocks, cols, counts = api.vertical_slash_select_lists(dev.q, dev.k, k_v, k_s)
    api.sparse_attn_lists(dev.q, dev.k, dev.v, blocks, counts, cols, out=out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        api.vertical_slash_select_lists(dev.q, dev.k, k_v, k_s, blocks=blocks, cols=cols, counts=counts)
        api.sparse_attn_lists(dev.q, dev.k, dev.v, blocks, counts, cols, out=out)
    e1.record()
    torch.cuda.synchronize()
    lms = e0.elapsed_time(e1) / reps
    _lib.profile_begin()
    api.vertical_slash_select_lists(dev.q, dev.k, k_v, k_s, blocks=blocks, cols=cols, counts=counts)
    api.sparse_attn_lists(dev.q, dev.k, dev.v, blocks, counts, cols, out=out)
    lprof = _lib.profile_end()
    cn = counts.to(torch.float64)
    res["vertical_slash"]["lists"] = dict(
        ms=lms, est_ms=sum(v[1] for k, v in lprof.items() if k.startswith("vs_")),
        attn_ms=sum(v[1] for k, v in lprof.items() if k.startswith("attn_")),
        index_bytes=(blocks.numel() + cols.numel() + counts.numel()) * 4,
        blocks_per_row=cn[..., 0].mean().item(), cols_per_row=cn[..., 1].mean().item())
    log(f"vertical-slash 128K, block and column lists: {lms:.2f} ms")
    del dev, out, blocks, cols, counts
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- #
# the other decode workloads: batch-32 ragged paged, and 3M tokens            #
# --------------------------------------------------------------------------- #
def other_decode(args, name, reps=24, n_queries=8, flush_bytes=1 << 30):
    """Graph-replayed decode step (dsa_prune_attend) of workload `name`, a
    fresh query each step, timed two ways: back to back (one KV copy, so later
    steps may find rows in the caches) and cache-cold (a 1 GiB read between
    steps, outside the timed region, evicts the L2s and the Infinity Cache;
    each step is timed alone with HIP events). HBM GB/s uses the algorithmic
    bytes of each step (SelectRep rows counted by the kernels + K/V rows of
    every kept key)."""
    import torch
    from dynamic_sparse_attention_query_amd import api, gen
    from dynamic_sparse_attention_query_amd.inputs import params_of, to_device

    t0 = time.time()
    case = gen.make_case(name, n_queries=n_queries)
    cfg = case.cfg
    dev = to_device(case)
    del case
    log(f"{name} inputs ready in {time.time() - t0:.1f}s")
    p = params_of(cfg)
    kw = dict(seq_lens=dev.seq_lens, block_table=dev.block_table, t=dev.t)
    qs = [dev.q[i].contiguous() for i in range(n_queries)]
    idx = torch.empty((cfg.batch, api._lib.index_width(p)), dtype=torch.int32, device="cuda")
    out = torch.empty(qs[0].shape, dtype=torch.float32, device="cuda")
    vis = torch.zeros(len(p.chunk), dtype=torch.int64, device="cuda")
    row_bytes = cfg.d * 2
    nbytes = []
    for q in qs:
        vis.zero_()
        api.prune_attend(q, dev.k, dev.v, p, idx=idx, out=out, visited=vis, **kw)
        torch.cuda.synchronize()
        nbytes.append(float(vis.sum().item()) * row_bytes + int((idx >= 0).sum().item()) * cfg.hkv * 2 * row_bytes)
    graphs = []
    for q in qs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            api.prune_attend(q, dev.k, dev.v, p, idx=idx, out=out, **kw)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    # back to back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        graphs[i % n_queries].replay()
    e1.record()
    torch.cuda.synchronize()
    us_b2b = e0.elapsed_time(e1) * 1e3 / reps
    # cache-cold: flush, then time one step. The flush reads a buffer larger
    # than the Infinity Cache, so the caches end holding clean lines (a write
    # would leave them dirty, and the timed step would pay for writing them
    # back).
    junk = torch.zeros(flush_bytes // 4, dtype=torch.float32, device="cuda")
    flush = torch.zeros((), dtype=torch.float32, device="cuda")
    torch.sum(junk, dim=0, out=flush)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        torch.sum(junk, dim=0, out=flush)
        evs[i][0].record()
        graphs[i % n_queries].replay()
        evs[i][1].record()
    torch.cuda.synchronize()
    us_cold = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / reps
    # the same per-step timing without the flush: separates the cache effect
    # from the cost of timing steps one at a time
    for i in range(reps):
        evs[i][0].record()
        graphs[i % n_queries].replay()
        evs[i][1].record()
        torch.cuda.synchronize()
    us_iso = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / reps
    nb = float(np.mean([nbytes[i % n_queries] for i in range(reps)]))

    def rate(us):
        g = nb / (us * 1e-6) / 1e9
        return round(g, 1), round(100 * g / PEAK_HBM_GBPS, 2)

    gb_cold, pct_cold = rate(us_cold)
    gb_b2b, pct_b2b = rate(us_b2b)
    res = {"us_per_step": round(us_cold, 2), "batch": cfg.batch, "us_per_token": round(us_cold / cfg.batch, 2),
           "algorithmic_bytes_per_step": int(nb), "gbps": gb_cold, "pct_peak": pct_cold,
           "timing": f"cache-cold: a {flush_bytes >> 30} GiB read between steps (outside the timed region), "
                     f"each step timed alone; {n_queries} distinct queries",
           "back_to_back": {"us_per_step": round(us_b2b, 2), "gbps": gb_b2b, "pct_peak": pct_b2b,
                            "timing": "back-to-back graph replays, distinct queries, one KV copy"},
           "isolated_warm_us_per_step": round(us_iso, 2),
           "tokens_in_context": int(dev.seq_lens.sum().item())}
    log(f"{name}: {us_cold:.1f} us/step cache-cold ({gb_cold} GB/s), {us_iso:.1f} isolated without flush, "
        f"{us_b2b:.1f} back to back")
    del dev, idx, out, graphs, junk, flush
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- #
# relative RoPE in SelectRep at the 1M decode shape                           #
# --------------------------------------------------------------------------- #
ROPE_BASE = 500000.0       # the rotary base of the Llama-3 shape
ROPE_STYLES = ("relative", "chunk_indexed")


def rope_decode(args, reps=20):
    """Graph-replayed 1M-token decode step (pruning + attention) with plain
    SelectRep and with each RoPE style inside it, on the same inputs:
    microseconds per step of each."""
    import torch
    from dynamic_sparse_attention_query_amd import api, gen
    from dynamic_sparse_attention_query_amd.inputs import params_of, to_device

    case = gen.make_case("c3", n_queries=1)
    cfg = case.cfg
    dev = to_device(case)
    del case
    p = params_of(cfg)
    q = dev.q[0].contiguous()
    kw = dict(seq_lens=dev.seq_lens, block_table=dev.block_table, t=dev.t)
    res = {}
    variants = [("plain", lambda out=None: api.prune_select(q, dev.k, p, out=out, **kw))]
    for style in ROPE_STYLES:
        variants.append((style, lambda out=None, style=style: api.prune_select_rope(q, dev.k, p, ROPE_BASE, out=out,
                                                                                     style=style, **kw)))
    # chunk-indexed over keys rotated once per stage: the whole context is
    # rotated before timing, and each timed step rotates the newest key (what
    # one appended token costs) and prunes over the rotated copies
    k_rot = api.rope_key_copies(dev.k, p)
    api.rope_rotate_keys(dev.k, p, ROPE_BASE, k_rot, seq_lens=dev.seq_lens)
    T = int(dev.k.shape[2])

    def prune_rotated_keys(out=None):
        api.rope_rotate_keys(dev.k, p, ROPE_BASE, k_rot, pos_begin=T - 1, pos_end=T, seq_lens=dev.seq_lens)
        return api.prune_select_rope_keys(q, k_rot, p, ROPE_BASE, seq_lens=dev.seq_lens, out=out)
    variants.append(("chunk_indexed_rotated_keys", prune_rotated_keys))
    for name, prune in variants:
        idx = prune()
        out = api.sparse_attn(q, dev.k, dev.v, idx, p, **kw)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            prune(out=idx.view(-1))
            api.sparse_attn(q, dev.k, dev.v, idx, p, out=out, **kw)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / reps
        res[name + "_idx"] = idx.clone()
        del g, out, idx
    plain_idx = res.pop("plain_idx")
    out = {"plain_us": round(res["plain"], 2),
           "note": "back-to-back graph replays of one step (same query, one KV copy)"}
    ci_idx = res["chunk_indexed_idx"].clone()
    for style in ROPE_STYLES:
        out[style] = {"us": round(res[style], 2), "overhead": round(res[style] / res["plain"], 3),
                      "index_row_changed": bool((res.pop(style + "_idx") != plain_idx).any().item())}
    rk = "chunk_indexed_rotated_keys"
    out[rk] = {"us": round(res[rk], 2), "overhead": round(res[rk] / res["plain"], 3),
               "same_rows_as_chunk_indexed": bool(torch.equal(res.pop(rk + "_idx"), ci_idx)),
               "note": "keys rotated once per stage (3 bf16 copies of K); each step rotates the newest key"}
    log("1M decode step: plain {:.1f} us, ".format(res["plain"]) +
        ", ".join(f"{st} RoPE {res[st]:.1f} us" for st in ROPE_STYLES) +
        f", chunk_indexed over rotated keys {res[rk]:.1f} us")
    del dev, k_rot
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- #
# CPU oracle baseline                                                         #
# --------------------------------------------------------------------------- #
# --------------------------------------------------------------------------- #
# CPU baseline: the oracle on the host's cores (a reported baseline only)     #
# --------------------------------------------------------------------------- #
_CPU_CASE = None             # the workload the pool workers read (inherited by fork)


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    global _CPU_LIMIT
    _CPU_LIMIT = threadpool_limits(limits=1)      # one BLAS thread per worker: parallelism is the pool


def _cpu_decode_step(qi):
    from oracle import ref
    case = _CPU_CASE
    cfg = case.cfg
    rp = ref.Params(1, cfg.chunk, cfg.keep, cfg.n_sink, cfg.n_window)
    T = cfg.t
    Q = case.q.sub((qi, 0))[:, None, :]
    row = ref.prune_block(Q, case.k[0], T - 1, T, rp)
    ref.attend_block(Q, case.k[0], case.v[0], row, T - 1, ref.default_scale(cfg.d))
    return qi


def _cpu_prefill_block(m):
    from oracle import ref
    case = _CPU_CASE
    cfg = case.cfg
    rp = ref.Params(cfg.block_q, cfg.chunk, cfg.keep, cfg.n_sink, cfg.n_window)
    s, e = m * cfg.block_q, (m + 1) * cfg.block_q
    Q = case.q.sub(0)[:, s:e]
    row = ref.prune_block(Q, case.k[0], s, e, rp)
    ref.attend_block(Q, case.k[0], case.v[0], row, s, ref.default_scale(cfg.d))
    return m


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args):
    """The oracle timed on the host's cores before the GPU is touched: a pool of
    worker processes (fork, one BLAS thread each) over distinct decode queries
    of the 1M workload, and over 64 stratified query blocks of the 128K prefill
    (every 32nd block), extrapolated to all blocks by the per-block flop model."""
    import multiprocessing as mp
    from dynamic_sparse_attention_query_amd import gen
    global _CPU_CASE
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("fork")
    res = {}
    _CPU_CASE = gen.make_case("c3")
    nq = _CPU_CASE.q.shape[0]
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_decode_step, range(workers))              # warm-up: page in the inputs
        t0 = time.perf_counter()
        done = pool.map(_cpu_decode_step, range(nq))
        el = time.perf_counter() - t0
    res["decode"] = {"value": round(el / len(done) * 1e6, 1), "unit": "us/token", "cores": workers,
                     "kind": "oracle", "cpu_model": _cpu_model(),
                     "sample": f"{len(done)} decode steps (distinct queries) of the 1M-token workload, oracle "
                               f"prune + attend, {workers} worker processes with one BLAS thread each, "
                               f"{el:.1f}s wall ({el * workers:.0f} worker-seconds)"}
    log(f"cpu oracle decode: {res['decode']['value']} us/token on {workers} workers")
    _CPU_CASE = gen.make_case("c2_128k")
    cfg = _CPU_CASE.cfg
    nblk = cfg.t // cfg.block_q
    blocks = list(range(nblk // 64 - 1, nblk, nblk // 64))      # 64 blocks, every 32nd, the last included
    sel, attn = prefill_block_flops(cfg)
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        t0 = time.perf_counter()
        pool.map(_cpu_prefill_block, blocks, chunksize=1)
        el = time.perf_counter() - t0
    flops = sel + attn
    sample_flops = float(flops[blocks].sum())
    ms = el * 1e3 * float(flops.sum()) / sample_flops
    res["prefill_128k"] = {"ms": round(ms, 1), "tflops": round(float(flops.sum()) / (ms * 1e-3) / 1e12, 4),
                           "cores": workers, "kind": "oracle", "extrapolated": True,
                           "sample": f"{len(blocks)} stratified query blocks (one in every {nblk // 64} of {nblk}) in "
                                     f"{el:.1f}s wall on {workers} workers, extrapolated to all blocks by the "
                                     f"per-block flop model (SelectRep evaluations + visible attention pairs)"}
    log(f"cpu oracle prefill 128K: {ms / 1e3:.1f} s extrapolated ({el:.1f}s for {len(blocks)} blocks)")
    _CPU_CASE = None
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} (WORLD_SIZE {world}) is not supported; "
              "the library runs on one GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    res = {}
    if not args.no_cpu:
        res["cpu"] = cpu_baseline(args)         # before the GPU is initialised (the pool forks)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_ref:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    case = decode_bench(args, res)
    if not args.no_other:
        res["c4"] = other_decode(args, "c4")
        res["c5"] = other_decode(args, "c5")
    if not args.no_prefill:
        prefill_bench(args, res)
    if not args.no_block_sparse:
        block_sparse_bench(args, res)
    if not args.no_vertical_slash:
        vertical_slash_bench(args, res)
    if not args.no_rope:
        res["rope_decode"] = rope_decode(args)

    dec = res["decode"]
    gbps = dec["bytes_per_step"] / (dec["us_per_step"] * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(dec["us_per_step"], 2),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["us_per_step"] / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c3-decode-1m: B=1, 32 q / 8 kv heads, d=128, T=1048576 bf16 grid K, N(0,1) V; "
                               "stages (l_c, k) = (256, 32768), (32, 8192), (8, 4096); 64 sink, 1024 window; "
                               "fresh query each step, 8 KV replicas cycled",
                   "global_batch": 1, "seq_len": 1048576, "parallelism": "none (1 GPU)"},
        "hbm_gbps": round(gbps, 1),
        "hbm_pct_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "algorithmic_bytes_per_step": int(dec["bytes_per_step"]),
        "selectrep_rows_per_stage": [round(x) for x in dec["stage_rows"]],
        "timing_mode": dec["mode"],
        "kernels_us": dec["kernels_us"],
        "roofline": dec["roofline"],
        "per_step_us": {"cache_cold": {"median": round(dec["per_step"]["cold"][0], 2),
                                       "p90": round(dec["per_step"]["cold"][1], 2),
                                       "mean": round(dec["per_step"]["cold"][2], 2)},
                        "isolated_warm": {"median": round(dec["per_step"]["warm"][0], 2),
                                          "p90": round(dec["per_step"]["warm"][1], 2),
                                          "mean": round(dec["per_step"]["warm"][2], 2)},
                        "timing": "64 steps (fresh query, KV replica cycled), each replayed alone between HIP "
                                  "events; cache-cold: a 1 GiB read before each step, outside the timed region"},
    }
    if "dense" in res:
        line["dense_decode_1m"] = {"us": round(res["dense"]["us"], 1), "gbps": round(res["dense"]["gbps"], 1),
                                   "pct_peak": round(100 * res["dense"]["gbps"] / PEAK_HBM_GBPS, 2),
                                   "sparse_speedup": round(res["dense"]["us"] / dec["us_per_step"], 2)}
    if "cached" in res:
        c = res["cached"]
        g = c["bytes_per_token"] / (c["us_per_token"] * 1e-6) / 1e9
        line["decode_cached_1m"] = {"refresh": c["refresh"], "us_per_token": round(c["us_per_token"], 2),
                                    "gbps": round(g, 1), "pct_peak": round(100 * g / PEAK_HBM_GBPS, 2),
                                    "algorithmic_bytes_per_token": int(c["bytes_per_token"]),
                                    "all_stages_due_step_us": round(c["full_refresh_step_us"], 2),
                                    "no_stage_due_step_us": round(c["reuse_step_us"], 2),
                                    "speedup_vs_uncached": round(dec["us_per_step"] / c["us_per_token"], 2)}
    if "c4" in res:
        line["decode_b32_paged_ragged"] = res["c4"]
    if "c5" in res:
        line["decode_3m"] = res["c5"]
    if "prefill" in res:
        pf = res["prefill"]
        line["prefill_128k"] = {"ms": round(pf["ms"], 2), "tflops": round(pf["tflops"], 2),
                                "pct_bf16_peak": round(100 * pf["tflops"] / PEAK_BF16_TFLOPS, 2),
                                "algorithmic_tflop": round(pf["algorithmic_tflop"], 2),
                                "selectrep_tflop": round(pf["selectrep_tflop"], 2),
                                "attn_tflop": round(pf["attn_tflop"], 2),
                                "prune_ms": round(pf["prune_ms"], 2), "attn_ms": round(pf["attn_ms"], 2),
                                "kernels_ms": pf["kernels_ms"]}
        kv = _counter_summary("prefill_128k_counters.md")
        if kv and "prefill_hbm_read_bytes" in kv:
            rb = int(kv["prefill_hbm_read_bytes"])
            line["prefill_128k"]["hbm_read_bytes_measured"] = rb
            line["prefill_128k"]["hbm_read_gbps"] = round(rb / (pf["ms"] * 1e-3) / 1e9, 1)
            line["prefill_128k"]["hbm_read_pct_peak"] = round(100 * rb / (pf["ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)
    if "block_sparse" in res:
        bs = res["block_sparse"]
        tf = bs["attn_tflop"] / (bs["ms"] * 1e-3)
        line["block_sparse_prefill_128k"] = {
            "k_blocks": BS_K_BLOCKS, "ms": round(bs["ms"], 2),
            "tflops": round(tf, 2), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "attn_tflop": round(bs["attn_tflop"], 2), "estimation_tflop_fp64": round(bs["est_tflop_fp64"], 3),
            "estimation_ms": round(bs["est_ms"], 3), "attn_ms": round(bs["attn_ms"], 2),
            "attn_only_pct_bf16_peak": round(100 * bs["attn_tflop"] / (bs["attn_ms"] * 1e-3) / PEAK_BF16_TFLOPS, 2),
            "dense_ms": round(bs["dense_ms"], 1) if bs["dense_ms"] else None,
            "speedup_vs_dense": round(bs["dense_ms"] / bs["ms"], 2) if bs["dense_ms"] else None,
            "kernels_ms": bs["kernels_ms"], "row_index_mb": round(bs["row_index_bytes"] / 1e6, 1)}
        if "lists" in bs:
            li = bs["lists"]
            line["block_sparse_prefill_128k"]["block_lists"] = {
                "ms": round(li["ms"], 2), "estimation_ms": round(li["est_ms"], 3), "attn_ms": round(li["attn_ms"], 2),
                "pct_bf16_peak": round(100 * bs["attn_tflop"] / (li["ms"] * 1e-3) / PEAK_BF16_TFLOPS, 2),
                "index_mb": round(li["index_bytes"] / 1e6, 1)}
        kv = _counter_summary("block_sparse_128k_counters.md")
        if kv and "bs_attn_fabric_read_bytes" in kv:
            rb = int(kv["bs_attn_fabric_read_bytes"])
            g = rb / (bs["attn_ms"] * 1e-3) / 1e9
            line["block_sparse_prefill_128k"]["attn_fabric_read_bytes_measured"] = rb
            line["block_sparse_prefill_128k"]["attn_fabric_read_gbps"] = round(g, 1)
            line["block_sparse_prefill_128k"]["attn_fabric_read_pct_hbm_peak"] = round(100 * g / PEAK_HBM_GBPS, 2)
    if "vertical_slash" in res:
        vs = res["vertical_slash"]
        tf = vs["attn_tflop"] / (vs["ms"] * 1e-3)
        dense_ms = res.get("block_sparse", {}).get("dense_ms")
        line["vertical_slash_prefill_128k"] = {
            "k_v": VS_KEEP[0], "k_s": VS_KEEP[1], "inputs": "c2 128K shape, keys along their own queries (local diagonal)",
            "ms": round(vs["ms"], 2), "tflops": round(tf, 2), "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "attn_tflop": round(vs["attn_tflop"], 2), "estimation_ms": round(vs["est_ms"], 3),
            "attn_ms": round(vs["attn_ms"], 2), "keys_per_row_mean": round(vs["entries"]), "row_width": vs["width"],
            "speedup_vs_dense": round(dense_ms / vs["ms"], 2) if dense_ms else None,
            "kernels_ms": vs["kernels_ms"], "row_index_mb": round(vs["row_index_bytes"] / 1e6, 1)}
        if "lists" in vs:
            li = vs["lists"]
            line["vertical_slash_prefill_128k"]["block_and_column_lists"] = {
                "ms": round(li["ms"], 2), "estimation_ms": round(li["est_ms"], 3), "attn_ms": round(li["attn_ms"], 2),
                "pct_bf16_peak": round(100 * vs["attn_tflop"] / (li["ms"] * 1e-3) / PEAK_BF16_TFLOPS, 2),
                "speedup_vs_dense": round(dense_ms / li["ms"], 2) if dense_ms else None,
                "index_mb": round(li["index_bytes"] / 1e6, 1), "blocks_per_row_mean": round(li["blocks_per_row"], 1),
                "cols_per_row_mean": round(li["cols_per_row"], 1)}
    if "rope_decode" in res or "rope_prefill" in res:
        rt = {"rotary_base": ROPE_BASE}
        if "rope_decode" in res:
            rt["decode_1m"] = res["rope_decode"]
        for style, r in res.get("rope_prefill", {}).items():
            rt.setdefault("prefill_128k", {"plain_ms": round(r["plain_ms"], 2),
                                           "plain_prune_ms": round(r["plain_prune_ms"], 2)})
            rt["prefill_128k"][style] = {"ms": round(r["ms"], 2), "prune_ms": round(r["prune_ms"], 2),
                                         "prune_overhead": round(r["prune_ms"] / r["plain_prune_ms"], 3),
                                         "rows_changed_fraction": round(r["rows_changed"], 4),
                                         "kernels_ms": r["kernels_ms"]}
        line["rope_in_selectrep"] = rt
    if "cpu" in res:
        line["cpu_baseline"] = res["cpu"]["decode"]
        line["cpu_baseline"]["prefill_128k"] = res["cpu"]["prefill_128k"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
