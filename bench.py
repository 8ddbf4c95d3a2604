#!/usr/bin/env python3
"""Throughput of the varlen GQA hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Default workload: long decode, B=1, Hq=64, Hkv=8 (G=8), D=128, one query
token over 32768 keys (split-KV: 32 splits x 8 KV heads = 256 workgroups).
A step is one execute of the plan (split kernel + merge) replayed from a
captured HIP graph of up to 40 steps, with inputs resident in HBM. K/V rotate
over enough copies (> 2x the 256 MB Infinity Cache) that every step reads from
HBM.

Prints ONE JSON line: value = KV GB/s over the K timed steps (whole job, one
GPU), roofline of the dominant kernel (algorithmic bytes per launch / mean
launch time from HIP events on its stream), the CPU oracle timed on a bounded
sample, and secondary measurements (causal varlen prefill TFLOP/s, batched
continuous-batching decode, padding mask) unless --no-secondary.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode KV GB/s (% of HBM peak) + µs/step; prefill TFLOP/s (% MFMA peak)"
MALL_DEFEAT_BYTES = 600 * 2**20


def _torch():
    import torch
    return torch


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

def time_replays(fn_list, steps, warmup):
    """Run fn_list[i % n] for warmup then `steps` iterations; returns
    (total ms for the timed steps, list of per-launch ms from event pairs)."""
    torch = _torch()
    n = len(fn_list)
    for i in range(warmup):
        fn_list[i % n]()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    for i in range(steps):
        fn_list[i % n]()
    t1.record(st)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    # per-launch event pairs (separate pass, same stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(st)
        fn_list[i % n]()
        evs[i][1].record(st)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return total, per


def kernel_event_times(plan, fn_list, steps):
    """Per-launch duration (ms) of the plan's main kernel over `steps` eager
    calls, from event pairs the library records around that kernel."""
    torch = _torch()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:  # create the HIP events
        a.record(st)
        b.record(st)
    torch.cuda.synchronize()
    n = len(fn_list)
    # the hook is set through the C entry point directly (event handles taken
    # beforehand), so the host stays ahead of the GPU and the kernels run back
    # to back as in a captured step
    import ctypes
    from varlen_gqa_attention_amd import _lib
    L = _lib.load()
    hs = [(ctypes.c_void_p(a.cuda_event), ctypes.c_void_p(b.cuda_event)) for a, b in evs]
    try:
        for i in range(steps):
            L.vattn_plan_set_kernel_events(plan._h, *hs[i])
            fn_list[i % n]()
    finally:
        plan.set_kernel_events(None, None)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def direct_calls(plan, q, ks, vs, cu_q, cu_kv, out, lse, B):
    """vattn_execute closures with their ctypes arguments built once (one per
    K/V copy): the same enqueue as Plan.__call__ without its per-call tensor
    checks, so that eager timing loops keep the GPU busy."""
    import ctypes
    torch = _torch()
    from varlen_gqa_attention_amd import _lib
    L = _lib.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = []
    for k, v in zip(ks, vs):
        a = (plan._h, B, P(q), P(k), P(v), P(cu_q), P(cu_kv), P(out), P(lse), q.shape[0],
             k.shape[0], st)
        calls.append(lambda a=a: _lib.check(L.vattn_execute(*a), "vattn_execute"))
    return calls


def capture(fn):
    torch = _torch()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        fn()
    torch.cuda.synchronize()
    return g


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key, digest):
    """Per-launch HBM bytes from the committed rocprofv3 counter summary, or
    None if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.lstrip().startswith("#"):
            continue
        parts = dict(p.split("=", 1) for p in line.split() if "=" in p)
        if parts.get("kernel") == kernel_key and parts.get("src") == digest:
            try:
                return float(parts["bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def long_decode(args):
    torch = _torch()
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    w = I.long_decode()
    B, Hq, Hkv, D, L = w["B"], w["Hq"], w["Hkv"], w["D"], int(w["kv_lens"][0])
    plan = V.Plan(B, 1, L, Hq, Hkv, D, False, **args.plan_opts)
    kv_bytes = 2 * L * Hkv * D * 2
    ncopy = max(1, -(-MALL_DEFEAT_BYTES // kv_bytes))
    q = I.normal_bf16((B, Hq, D), 10, "cuda")
    ks = [I.normal_bf16((L, Hkv, D), 11 + 2 * i, "cuda") for i in range(ncopy)]
    vs = [I.normal_bf16((L, Hkv, D), 12 + 2 * i, "cuda") for i in range(ncopy)]
    cu_q = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    cu_kv = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, device="cuda")
    fns = []
    for i in range(ncopy):
        k, v = ks[i], vs[i]
        fns.append(lambda k=k, v=v: plan(q, k, v, cu_q, cu_kv, out=out, lse=lse, B=B))
    graphs = [capture(f) for f in fns]
    # one graph holds gsteps consecutive steps (one per K/V copy, in turn), as
    # a model's captured decode forward holds one attention call per layer
    # (up to 40 here); each graph replay adds a fixed ~5 us boundary, which a
    # short graph would charge to few steps
    gsteps = args.graph_steps if args.graph_steps > 0 else min(40, max(ncopy, args.steps))
    if gsteps > 1:
        group = capture(lambda: [fns[i % ncopy]() for i in range(gsteps)])
        seq = [group.replay] * (args.steps // gsteps) + \
              [graphs[i % ncopy].replay for i in range(args.steps % gsteps)]
        for i in range(max(1, args.warmup // gsteps)):
            group.replay()
        torch.cuda.synchronize()
        total, _ = time_replays(seq, len(seq), 0)
        # the median step: 50 replays of the graph, event pair around each
        _, per_rep = time_replays([group.replay], 50, 2)
        med_step_ms = sorted(per_rep)[len(per_rep) // 2] / gsteps
        n_med = len(per_rep)
    else:
        total, per_rep = time_replays([g.replay for g in graphs], args.steps, args.warmup)
        med_step_ms = sorted(per_rep)[len(per_rep) // 2]
        n_med = len(per_rep)
    # execute-level event pairs (split + merge), eager, same stream
    direct = direct_calls(plan, q, ks, vs, cu_q, cu_kv, out, lse, B)
    _, per = time_replays(direct, args.steps, 5)
    # the dominant kernel alone: the library records an event pair right
    # around the split kernel of every eager execute (measurement hook)
    kern = kernel_event_times(plan, direct, args.steps)
    ms = total / args.steps
    alg_bytes = kv_bytes + 2 * B * Hq * D * 2 + B * Hq * 4   # K+V, Q, O, LSE
    split_bytes = kv_bytes + B * Hq * D * 2                  # K+V, Q
    mean_exec_ms = sum(per) / len(per)
    mean_kern_ms = sum(kern) / len(kern)
    info = plan.info
    src = ["varlen_gqa_attention_amd/csrc/decode.hip", "varlen_gqa_attention_amd/csrc/device.hpp"]
    digest = source_digest(src)
    traffic = stored_traffic("decode_long", digest)
    res = dict(
        metric=METRIC, value=round(kv_bytes / (ms * 1e-3) / 1e9, 1), unit="GB/s",
        ms_per_step=round(ms, 5), us_per_step=round(ms * 1e3, 2),
        us_per_step_median=round(med_step_ms * 1e3, 2),
        median_note=f"median over {n_med} replays of the {gsteps}-step graph (event pair around "
                    "each), per step",
        kv_bytes_per_step=kv_bytes, frac_hbm_peak=round(kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        config=dict(workload="long decode: B=1, Hq=64, Hkv=8, D=128, Lk=32768, bf16 THD, "
                             f"{ncopy} rotating K/V copies (MALL defeat), graphs of {gsteps} step(s)",
                    B=B, Hq=Hq, Hkv=Hkv, D=D, kv_len=L, nsplit=info["nsplit"],
                    decode_path=("mfma" if info["decode_path"] == 2 else "wave"),
                    grid=info["grid"], threads=info["threads"],
                    fused_combine=info["fused_combine"]),
        roofline=dict(bound="hbm", achieved=round(split_bytes / (mean_kern_ms * 1e-3) / 1e9, 1),
                      peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(split_bytes / (mean_kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      traffic=traffic,
                      kernel=f"decode_{'mfma' if info['decode_path'] == 2 else 'wave'}_kernel "
                             "(split-KV pass; K, V and Q bytes)",
                      bytes_per_launch=split_bytes, mean_launch_us=round(mean_kern_ms * 1e3, 2),
                      median_launch_us=round(sorted(kern)[len(kern) // 2] * 1e3, 2),
                      timing=f"HIP events around the kernel, {len(kern)} eager executes",
                      src_digest=digest),
        execute=dict(bytes=alg_bytes, mean_us=round(mean_exec_ms * 1e3, 2),
                     gbs=round(alg_bytes / (mean_exec_ms * 1e-3) / 1e9, 1),
                     note="one eager execute (split + LSE combine), HIP events on its stream"),
    )
    state = dict(plan=plan, q=q, k=ks[0], v=vs[0], cu_q=cu_q, cu_kv=cu_kv, B=B, L=L)
    return res, state


def shard_decode_measure(args, reps=10):
    """One GPU's share of the long decode under KV-head sharding over 8 GPUs
    (B=1, Hq=8, Hkv=1, D=128, Lk=32768): graph-replayed step time with the
    default plan (split cap 32 and 1024-key minimum chunk: 32 workgroups) and
    with the split count forced so that the grid fills the CUs."""
    torch = _torch()
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    B, Hq, Hkv, D, L = 1, 8, 1, 128, 32768
    kv_bytes = 2 * L * Hkv * D * 2
    ncopy = max(1, -(-MALL_DEFEAT_BYTES // kv_bytes))
    q = I.normal_bf16((B, Hq, D), 20, "cuda")
    ks = [I.normal_bf16((L, Hkv, D), 21 + 2 * i, "cuda") for i in range(ncopy)]
    vs = [I.normal_bf16((L, Hkv, D), 22 + 2 * i, "cuda") for i in range(ncopy)]
    cu_q = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    cu_kv = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, device="cuda")
    res = dict(workload=f"one GPU's share of the long decode at 8-way head sharding: B=1, "
                        f"Hq=8, Hkv=1, D=128, Lk=32768, {ncopy} rotating K/V copies, graphs of "
                        f"{ncopy} steps", kv_bytes_per_step=kv_bytes)
    for name, opts in (("default_plan", {}), ("forced_128_splits", dict(force_nsplit=128)),
                       ("forced_256_splits", dict(force_nsplit=256))):
        plan = V.Plan(B, 1, L, Hq, Hkv, D, False, **opts)
        fns = [lambda k=k, v=v: plan(q, k, v, cu_q, cu_kv, out=out, lse=lse, B=B)
               for k, v in zip(ks, vs)]
        group = capture(lambda: [f() for f in fns])
        total, _ = time_replays([group.replay], reps, 2)
        us = total / (reps * ncopy) * 1e3
        res[name] = dict(nsplit=plan.info["nsplit"], grid=plan.info["grid"],
                         us_per_step=round(us, 2),
                         kv_gbs=round(kv_bytes / (us * 1e-6) / 1e9, 1))
    return res


def cold_step_times(step, reps, flush_bytes=640 * 2**20):
    """Per-step GPU time (HIP events on the stream) of `step` with the
    Infinity Cache and L2 emptied of its inputs before each step: a read of
    a buffer larger than twice the 256 MB Infinity Cache runs between steps,
    outside the event pair (a read leaves no dirty lines to write back)."""
    torch = _torch()
    scrub = torch.ones(flush_bytes // 4, device="cuda")
    sink = torch.empty((), device="cuda")
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for _ in range(3):
        step()
    for a, b in evs:
        torch.sum(scrub, dim=0, out=sink)
        a.record(st)
        step()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def small_configs_measure(reps=200):
    """The two remaining decode configurations, graph-replayed: the tiny
    decode (B=2, Hq=4, Hkv=1, D=64, KV lengths U[1,128] seed (0,0)), which is
    latency-bound and reported in µs/step, and the edge sweep (B=33 of
    B_max=64, Hq=128, Hkv=8, lengths 0..16384, adversarial cu tails) at
    D = 32, 64 and 256, in µs/step and GB/s of K+V read."""
    torch = _torch()
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    res = {}
    for w in [I.tiny_decode(0)] + [I.edge_sweep(D) for D in (32, 64, 256)]:
        m = I.materialise(w, 0, "cuda")
        plan = V.Plan(w["B_max"], 1, w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], False)
        out = torch.empty_like(m["q"])
        lse = torch.empty(m["q"].shape[:2], device="cuda")
        f = lambda: plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], out=out, lse=lse,
                         B=w["B"])
        per_graph = 10   # steps per graph, so that host graph launches stay off the clock
        g = capture(lambda: [f() for _ in range(per_graph)])
        total, _ = time_replays([g.replay], reps // per_graph, 2)
        us = total / (reps // per_graph * per_graph) * 1e3
        # cold: one step per graph replay, caches emptied of the inputs first
        g1 = capture(f)
        cold = cold_step_times(g1.replay, 50)
        us_cold = sorted(cold)[len(cold) // 2] * 1e3
        kv = int(2 * w["kv_lens"].sum() * w["Hkv"] * w["D"] * 2)
        res[w["name"]] = dict(us_per_step_cold=round(us_cold, 2),
                              kv_gbs_cold=round(kv / (us_cold * 1e-6) / 1e9, 1),
                              us_per_step_warm=round(us, 2),
                              kv_gbs_warm=round(kv / (us * 1e-6) / 1e9, 1), kv_bytes=kv,
                              nsplit=plan.info["nsplit"], grid=plan.info["grid"],
                              fused_combine=plan.info["fused_combine"],
                              decode_path=("mfma" if plan.info["decode_path"] == 2 else "wave"))
        plan.close()
    res["note"] = ("cold: median of 50 single-step graph replays, each after a 640 MiB read "
                   "that empties the Infinity Cache and L2 of the step's inputs (HIP events "
                   "around the step only); warm: graphs of 10 back-to-back steps on resident "
                   "K/V (the edge sweep's K/V fit in the 256 MB Infinity Cache at D = 32 and "
                   "64, so those warm rates are cache-assisted)")
    return res


def cpu_baseline_long_decode(state, budget_s):
    import numpy as np
    from oracle import attention as A
    from varlen_gqa_attention_amd import inputs as I
    q = I.bf16_to_f64(state["q"])
    k = I.bf16_to_f64(state["k"])
    v = I.bf16_to_f64(state["v"])
    L = state["L"]
    B = state["B"]
    cu_q, cu_kv = np.array([0, 1]), np.array([0, L])
    t0 = time.perf_counter()
    n = 0
    while True:
        A.attend_varlen(q, k, v, cu_q, cu_kv, B, False)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    kv_bytes = 2 * L * k.shape[1] * k.shape[2] * 2
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    cores = min(len(os.sched_getaffinity(0)), max(1, blas))
    return dict(value=round(kv_bytes / dt / 1e9, 3), unit="GB/s", cores=cores, kind="oracle",
                sample=f"{n} full long-decode step(s) of the fp64 NumPy oracle "
                       f"({dt:.2f} s each; K/V of bf16 values copied to host, untimed)")


def cpu_baseline_prefill(budget_s):
    """The oracle's forward and backward on one (sequence, query head) of the
    causal varlen prefill workload (its longest sequence), as GFLOP/s of the
    same algorithmic flop counts the GPU lines use (4 D and 8 D per visible
    pair): the bounded sample of the prefill and backward rows."""
    import numpy as np
    from oracle import attention as A
    from oracle import backward as BW
    from varlen_gqa_attention_amd import inputs as I
    w = I.varlen_prefill(0)
    L = int(np.max(w["q_lens"]))
    D = w["D"]
    rng = np.random.default_rng(0)   # values of the sample (the timing does not depend on them)
    q, k, v, do = (rng.standard_normal((L, D)) for _ in range(4))
    vis = A.visible_keys(L, L, True)
    pairs = int(vis.sum())
    scale = 1.0 / np.sqrt(D)
    out = {}
    for name, fn, flop in (("prefill", lambda: A.attend_rows(q, k, v, vis, scale), 4 * D * pairs),
                           ("backward", lambda: BW.backward_rows(q, k, v, do, vis, scale),
                            8 * D * pairs)):
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / n
        out[name] = dict(value=round(flop / dt / 1e9, 2), unit="GFLOP/s",
                         sample=f"{n} call(s) on one query head of a {L}-token causal sequence "
                                f"({dt:.2f} s each)")
    return out


def cpu_baseline_configs(prefill_rate_gflops=None):
    """The oracle timed on each remaining configuration (seconds per step on
    the host, bounded samples): the tiny decode (whole step, repeated for
    about a second), the edge sweep at D = 32, 64 and 256 (one whole step
    each), the continuous-batching decode (steps 0 and 1 of its 100; the
    lengths differ per step), and the causal varlen prefill extrapolated from
    the one-head sample's GFLOP/s to the workload's algorithmic flops. Values
    are drawn on the host (the timing does not depend on them)."""
    import numpy as np
    from oracle import attention as A
    from varlen_gqa_attention_amd import inputs as I
    out = {}

    def time_step(w, seed, min_s=0.0):
        m = I.materialise(w, seed, "cpu")
        q, k, v = (I.bf16_to_f64(m[n]) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        n = 0
        while True:
            A.attend_varlen(q, k, v, m["cu_q_np"], m["cu_kv_np"], w["B"], w["causal"])
            n += 1
            if time.perf_counter() - t0 >= min_s:
                break
        return (time.perf_counter() - t0) / n, n

    dt, n = time_step(I.tiny_decode(0), 0, min_s=1.0)
    out["tiny decode"] = dict(s_per_step=round(dt, 5), sample=f"{n} whole steps")
    for D in (32, 64, 256):
        w = I.edge_sweep(D)
        dt, n = time_step(w, D)
        out[w["name"]] = dict(s_per_step=round(dt, 3), sample="one whole step")
    ts = []
    for t in (0, 1):
        dt, _ = time_step(I.batched_decode_step(t), t)
        ts.append(dt)
    out["continuous-batching decode"] = dict(
        s_per_step=round(sum(ts) / len(ts), 3),
        sample="steps 0 and 1 of the 100 (lengths U[128, 8192] each), mean")
    if prefill_rate_gflops:
        w = I.varlen_prefill(0)
        flop = 4 * w["Hq"] * w["D"] * visible_pairs(w["q_lens"], w["kv_lens"])
        out["causal varlen prefill"] = dict(
            s_per_step=round(flop / (prefill_rate_gflops * 1e9), 1),
            sample="extrapolated: the workload's algorithmic flops at the GFLOP/s the oracle "
                   "reached on one query head of its longest sequence")
    return out


def visible_pairs(q_lens, kv_lens):
    """(query, key) pairs a causal (bottom-right aligned) pass must compute:
    query i of a sequence sees keys j <= i + Lk - Lq, clamped to [0, Lk)."""
    total = 0
    for lq, lk in zip(q_lens, kv_lens):
        lq, lk = int(lq), int(lk)
        shift = lk - lq
        # rows i with i + shift + 1 in [0, lk]: count min(lk, max(0, i + shift + 1))
        for i in range(lq):
            total += min(lk, max(0, i + shift + 1))
    return total


def prefill_measure(args, reps=10):
    torch = _torch()
    import numpy as np
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    w = I.varlen_prefill(0)
    if getattr(args, "prefill_len", 0):
        # profiling aid: every sequence at the same length (not the headline workload)
        w["q_lens"] = w["kv_lens"] = np.full(w["B"], args.prefill_len, dtype=np.int64)
        w["name"] += f" (all lengths {args.prefill_len})"
    m = I.materialise(w, 0, "cuda")
    plan = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], True)
    plan_p = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], True,
                    prefill_grid=1)
    out = torch.empty_like(m["q"])
    lse = torch.empty(m["q"].shape[:2], device="cuda")
    pairs = visible_pairs(w["q_lens"], w["kv_lens"])
    flop = 4 * w["Hq"] * w["D"] * pairs
    med = lambda xs: sorted(xs)[len(xs) // 2]
    # default: grid from B_max and s_max_q, dead tiles exit (one kernel)
    f = lambda: plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], out=out, lse=lse, B=w["B"])
    # bring the clocks up before the first timed variant (about 0.5 s of work)
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        f()
        torch.cuda.synchronize()
    _, per = time_replays([f], reps, 2)
    ms = med(per)
    kern = kernel_event_times(plan, [f], reps)
    # device-built live-tile schedule + persistent grid (two kernels)
    fp = lambda: plan_p(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], out=out, lse=lse, B=w["B"])
    _, per_p = time_replays([fp], reps, 2)
    tq = plan.info["q_tokens_per_tile"]
    # exact grid: live tiles only, longest first (host knows lengths here)
    lens = w["q_lens"]
    tiles = sorted(((b << 16) | t for b, L in enumerate(lens) for t in range(-(-int(L) // tq))),
                   key=lambda e: -(e & 0xFFFF))
    tmap = torch.tensor(tiles, dtype=torch.int32, device="cuda")
    fe = lambda: plan.execute_exact_grid(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], tmap,
                                           out, lse, w["B"])
    _, per_e = time_replays([fe], reps, 2)

    # declared strides: q, k, v as slices of one fused QKV buffer, out as a
    # slice of a wider buffer (no copies; same kernel, strided addressing)
    Tq = m["q"].shape[0]
    qkv = torch.empty(Tq, w["Hq"] + 2 * w["Hkv"], w["D"], dtype=torch.bfloat16, device="cuda")
    qkv[:, :w["Hq"]] = m["q"]
    qkv[:, w["Hq"]:w["Hq"] + w["Hkv"]] = m["k"]
    qkv[:, w["Hq"] + w["Hkv"]:] = m["v"]
    wide = torch.empty(Tq, w["Hq"] + 8, w["D"], dtype=torch.bfloat16, device="cuda")
    qs, ks_, vs_ = qkv[:, :w["Hq"]], qkv[:, w["Hq"]:w["Hq"] + w["Hkv"]], qkv[:, w["Hq"] + w["Hkv"]:]
    fs = lambda: plan(qs, ks_, vs_, m["cu_q"], m["cu_kv"], out=wide[:, :w["Hq"]], lse=lse, B=w["B"])
    _, per_s = time_replays([fs], reps, 2)

    def roundtrip():  # the D2H + host cumsum + H2D path the grid-sizing issue describes
        lens_h = (m["cu_q"][1:w["B"] + 1] - m["cu_q"][:w["B"]]).cpu().numpy()
        tl = [(b << 16) | t for b, L in enumerate(lens_h) for t in range(-(-int(L) // tq))]
        tm = torch.tensor(tl, dtype=torch.int32).to("cuda", non_blocking=False)
        plan.execute_exact_grid(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], tm, out, lse,
                                w["B"])
    _, per_r = time_replays([roundtrip], reps, 2)
    tfl = flop / (ms * 1e-3) / 1e12
    kfl = flop / (med(kern) * 1e-3) / 1e12
    return dict(workload=w["name"] + ": B=16, L~U[64,4096] (seed 3,0), Hq=32, Hkv=8, "
                         "D=128, s_max 4096", flop=flop, causal_pairs=pairs,
                us=round(ms * 1e3, 1), tflops=round(tfl, 1),
                frac_mfma_peak=round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                timing=f"median of {reps} eager executes, HIP events on the stream",
                grid=plan.info["grid"], schedule="grid from B_max and s_max_q, dead tiles exit",
                kernel_us=round(med(kern) * 1e3, 1), kernel_tflops=round(kfl, 1),
                live_tiles=len(tiles) * w["Hkv"],
                scheduled_persistent_us=round(med(per_p) * 1e3, 1),
                exact_grid_us=round(med(per_e) * 1e3, 1),
                fused_qkv_strided_us=round(med(per_s) * 1e3, 1),
                exact_grid_with_host_roundtrip_us=round(med(per_r) * 1e3, 1))


def backward_measure(args, reps=10):
    """Backward (dq, dk, dv) on the causal varlen prefill workload: the
    forward's out and lse feed it, dout is seeded N(0, 1) bf16. Algorithmic
    flop = 8 * Hq * D per visible pair (the four length-D products dv, dp, dq,
    dk of each pair); the kernels also recompute S and dP in both passes."""
    torch = _torch()
    import numpy as np
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    w = I.varlen_prefill(0)
    if getattr(args, "prefill_len", 0):
        w["q_lens"] = w["kv_lens"] = np.full(w["B"], args.prefill_len, dtype=np.int64)
        w["name"] += f" (all lengths {args.prefill_len})"
    m = I.materialise(w, 0, "cuda")
    plan = V.Plan(w["B_max"], w["s_max_q"], w["s_max_kv"], w["Hq"], w["Hkv"], w["D"], True,
                  backward=True)
    out, lse = plan(m["q"], m["k"], m["v"], m["cu_q"], m["cu_kv"], B=w["B"])
    dout = I.normal_bf16(tuple(m["q"].shape), 77, "cuda")
    dq, dk, dv = torch.empty_like(m["q"]), torch.empty_like(m["k"]), torch.empty_like(m["v"])
    pairs = visible_pairs(w["q_lens"], w["kv_lens"])
    flop = 8 * w["Hq"] * w["D"] * pairs
    med = lambda xs: sorted(xs)[len(xs) // 2]
    f = lambda: plan.backward(m["q"], m["k"], m["v"], out, lse, dout, m["cu_q"], m["cu_kv"],
                              dq=dq, dk=dk, dv=dv, B=w["B"])
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        f()
        torch.cuda.synchronize()
    _, per = time_replays([f], reps, 2)
    ms = med(per)
    kern = kernel_event_times(plan, [f], reps)
    tfl = flop / (ms * 1e-3) / 1e12
    return dict(workload=w["name"] + ": backward, B=16, L~U[64,4096] (seed 3,0), Hq=32, Hkv=8, "
                         "D=128, s_max 4096",
                flop=flop, flop_rule="8 * Hq * D per visible (query, key) pair",
                us=round(ms * 1e3, 1), tflops=round(tfl, 1),
                frac_mfma_peak=round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                kernels_us=round(med(kern) * 1e3, 1),
                grids=dict(dq=plan.info["bwd_grid_dq"], dkdv=plan.info["bwd_grid_dkdv"]),
                timing=f"median of {reps} eager calls (dq kernel + dk/dv kernel), HIP events")


def batched_decode_measure(args, steps=100, split_rule=None):
    torch = _torch()
    import numpy as np
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    ws = [I.batched_decode_step(t) for t in range(steps)]
    w = ws[0]
    B, Hq, Hkv, D, smax = w["B"], w["Hq"], w["Hkv"], w["D"], w["s_max_kv"]
    opts = dict(args.plan_opts)
    if split_rule is not None:
        opts.pop("target_blocks_per_cu", None)
        opts["split_rule"] = split_rule
    plan = V.Plan(B, 1, smax, Hq, Hkv, D, False, **opts)
    pool = B * smax  # room for B sequences of s_max rows: 1 GiB per K/V tensor
    q = I.normal_bf16((B, Hq, D), 20, "cuda")
    k = I.normal_bf16((pool, Hkv, D), 21, "cuda")
    v = I.normal_bf16((pool, Hkv, D), 22, "cuda")
    # per-step offsets: sequence b starts at b * smax (+ a per-step shift) with length L_b
    cus = []
    kv_bytes = []
    for t, wt in enumerate(ws):
        # this step's sequences packed back to back from the start of the pool
        cu = np.concatenate([[0], np.cumsum(wt["kv_lens"])]).astype(np.int32)
        cus.append(cu)
        kv_bytes.append(int(wt["kv_lens"].sum()) * Hkv * D * 2 * 2)
    cu_all = torch.from_numpy(np.stack(cus)).cuda()
    cu_rows = [cu_all[t] for t in range(steps)]  # contiguous rows, one per step
    cu_q = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, device="cuda")
    st = torch.cuda.current_stream()

    # the 100 steps back to back in one captured graph, each step reading its
    # own cu_seqlens row: mean time per step
    def all_steps():
        for t in range(steps):
            plan(q, k, v, cu_q, cu_rows[t], out=out, lse=lse, B=B)
    g_all = capture(all_steps)
    g_all.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    g_all.replay()
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # one graph per step, events around each replay: the median step
    gs = [capture(lambda t=t: plan(q, k, v, cu_q, cu_rows[t], out=out, lse=lse, B=B))
          for t in range(steps)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for g1, (a, b) in zip(gs, evs):
        a.record(st)
        g1.replay()
        b.record(st)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    # the capture-once form: one graph of {select this step's cu on the device,
    # execute, advance the step counter} replayed 100 times (includes the
    # selection and counter kernels)
    live = torch.zeros(1, B + 1, dtype=torch.int32, device="cuda")
    step = torch.zeros(1, dtype=torch.int64, device="cuda")

    def one():
        torch.index_select(cu_all, 0, step, out=live)
        plan(q, k, v, cu_q, live.view(-1), out=out, lse=lse, B=B)
        step.add_(1)
    g = capture(one)
    step.zero_()
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(st)
    t_host0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    t_host1 = time.perf_counter()
    e3.record(st)
    torch.cuda.synchronize()
    ms_counter = e2.elapsed_time(e3) / steps
    assert int(step.item()) == steps
    mean_bytes = sum(kv_bytes) / steps
    info = plan.info
    return dict(workload="continuous-batching decode: B=64, Hq=32, Hkv=8, D=128, s_max_kv=8192, "
                         "lengths U[128,8192] per step (seed 2,t), 100 steps in one captured graph",
                split_rule=split_rule or "default",
                us_per_step=round(ms * 1e3, 1), kv_gbs=round(mean_bytes / (ms * 1e-3) / 1e9, 1),
                us_per_step_median=round(per[len(per) // 2] * 1e3, 1),
                median_note="one graph per step, HIP events around each replay",
                frac_hbm_peak=round(mean_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                us_per_step_device_counter=round(ms_counter * 1e3, 1),
                device_counter_note="one graph of {index_select of the step's cu row, execute, "
                                    "step += 1} replayed 100 times",
                host_enqueue_us_per_step=round((t_host1 - t_host0) / steps * 1e6, 1),
                decode_path=("mfma" if info["decode_path"] == 2 else "wave"),
                nsplit=info["nsplit"], direct=info["direct"], fused_combine=info["fused_combine"],
                grid=info["grid"])


def mask_measure():
    torch = _torch()
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    lens = I.edge_sweep_lengths(64)
    cu = torch.from_numpy(I.cu_from_lengths(lens, 65, [-1, 2**31 - 1, int(lens.sum())])).cuda()
    out = torch.empty((33, 1, 1, 16384), dtype=torch.bool, device="cuda")
    f = lambda: V.padding_mask(cu, 33, 16384, out=out)
    _, per = time_replays([f], 50, 5)
    # cross attention: query-side and key-side masks in one launch (key
    # lengths: the same values in reverse order)
    cu_k = torch.from_numpy(I.cu_from_lengths(lens[::-1].copy(), 65,
                                              [-1, 2**31 - 1, int(lens.sum())])).cuda()
    out_k = torch.empty_like(out)
    fc = lambda: V.cross_padding_masks(cu, cu_k, 33, 16384, 16384, out_q=out, out_kv=out_k)
    _, per_c = time_replays([fc], 50, 5)
    return dict(workload="padding mask B=33, max_seqlen=16384 (540672 bytes)",
                us=round(sorted(per)[len(per) // 2] * 1e3, 2),
                cross_us=round(sorted(per_c)[len(per_c) // 2] * 1e3, 2),
                cross_workload="query-side and key-side masks, B=33, 16384 each (1081344 bytes)")


def gathered_measure(steps=50, **plan_opts):
    """Decode over gathered keys: 16 sequences, each attending 2048 rows
    selected (sorted, without repeats) from its own 32768-token history."""
    torch = _torch()
    import numpy as np
    import varlen_gqa_attention_amd as V
    from varlen_gqa_attention_amd import inputs as I
    B, Hq, Hkv, D, hist, sel = 16, 32, 8, 128, 32768, 2048
    plan = V.Plan(B, 1, sel, Hq, Hkv, D, False, **plan_opts)
    q = I.normal_bf16((B, Hq, D), 40, "cuda")
    k = I.normal_bf16((B * hist, Hkv, D), 41, "cuda")
    v = I.normal_bf16((B * hist, Hkv, D), 42, "cuda")
    rng = I.rng(7, 0)
    idx = np.concatenate([b * hist + np.sort(rng.choice(hist, sel, replace=False))
                          for b in range(B)]).astype(np.int32)
    kv_idx = torch.from_numpy(idx).cuda()
    cu_q = torch.from_numpy(I.cu_from_lengths(np.ones(B, np.int64))).cuda()
    cu_idx = torch.from_numpy(I.cu_from_lengths(np.full(B, sel))).cuda()
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, device="cuda")
    f = lambda: plan.gathered(q, k, v, cu_q, cu_idx, kv_idx, out=out, lse=lse, B=B)
    g = capture(f)
    total, _ = time_replays([g.replay], steps, 5)
    ms = total / steps
    kv_bytes = B * sel * Hkv * D * 2 * 2
    return dict(workload=f"gathered-key decode: B={B}, Hq={Hq}, Hkv={Hkv}, D={D}, {sel} keys per "
                         f"sequence selected from {hist} (sorted, seed 7), graph replay",
                us_per_step=round(ms * 1e3, 2), kv_gbs=round(kv_bytes / (ms * 1e-3) / 1e9, 1),
                frac_hbm_peak=round(kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                nsplit=plan.info["nsplit"],
                decode_path=("mfma" if plan.info["decode_path"] == 2 else "wave"))


def calibrate_copy():
    """Plain elementwise copy of a known size, for scaling HBM counters."""
    torch = _torch()
    n = 256 * 2**20 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n * 4, "bytes_written": n * 4}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--force-nsplit", type=int, default=0)
    ap.add_argument("--decode-path", type=int, default=0, choices=[0, 1, 2])
    ap.add_argument("--fuse-combine", type=int, default=0, choices=[0, 1, 2])
    ap.add_argument("--nsplit-cap", type=int, default=0)
    ap.add_argument("--target-blocks", type=int, default=0,
                    help="decode split rule: workgroups per CU to aim for (0 = plan default)")
    ap.add_argument("--prefill-len", type=int, default=0,
                    help="with --workload prefill: give every sequence this length")
    ap.add_argument("--decode-waves", type=int, default=0, choices=[0, 4, 8])
    ap.add_argument("--split-rule", default=None, choices=["default", "pages"],
                    help="with --workload batched_decode: the decode split rule")
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="long decode: steps per captured graph (0 = min(40, --steps))")
    ap.add_argument("--workload", default="long_decode",
                    choices=["long_decode", "prefill", "batched_decode", "gathered_decode",
                             "backward", "shard_decode", "small_configs"],
                    help="headline workload (default: long decode); the others are for "
                         "profiling runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 (sharding across GPUs is "
                                   "not implemented)"}))
        sys.exit(2)
    args.plan_opts = dict(target_blocks_per_cu=args.target_blocks,
                          force_nsplit=args.force_nsplit, force_decode_path=args.decode_path,
                          fuse_combine=args.fuse_combine, nsplit_cap=args.nsplit_cap,
                          decode_waves=args.decode_waves)
    torch = _torch()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload == "gathered_decode":
        print(json.dumps({"workload": args.workload,
                          **gathered_measure(**{k: v for k, v in args.plan_opts.items() if v})}))
        return
    if args.workload != "long_decode":
        fn = {"prefill": prefill_measure, "backward": backward_measure,
              "shard_decode": shard_decode_measure,
              "small_configs": lambda _args: small_configs_measure()}.get(
                  args.workload,
                  lambda a: batched_decode_measure(a, split_rule=a.split_rule))
        print(json.dumps({"workload": args.workload, **fn(args)}))
        return
    res, state = long_decode(args)
    line = dict(metric=res.pop("metric"), value=res.pop("value"), unit=res.pop("unit"),
                n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=res.pop("ms_per_step"), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16", data="synthetic")
    line.update(res)
    if not args.no_secondary:
        line["prefill"] = prefill_measure(args)
        line["batched_decode"] = batched_decode_measure(args)
        line["batched_decode_pages_rule"] = batched_decode_measure(args, split_rule="pages")
        line["gathered_decode"] = gathered_measure()
        line["backward"] = backward_measure(args)
        line["shard_decode"] = shard_decode_measure(args)
        line["small_configs"] = small_configs_measure()
        line["padding_mask"] = mask_measure()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_long_decode(state, args.cpu_budget)
        if not args.no_secondary:
            sec = cpu_baseline_prefill(min(5.0, args.cpu_budget))
            line["cpu_baseline"]["secondary"] = sec
            line["cpu_baseline"]["per_config"] = cpu_baseline_configs(sec["prefill"]["value"])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()
