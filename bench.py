#!/usr/bin/env python3
"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

One step = layout (counts, aligned offsets, stable slots, per-rank token sets)
and dispatch scatter in one call (moe_layout_dispatch), then combine
(moe_combine; identity expert: the combine reads the receive buffer the
dispatch wrote) for one batch of the standard workload: 128 tokens
x 7168 hidden bf16, 256 experts on 8 logical ranks, top-8 uniform routing,
softmax weights. Inputs are seeded and synthetic and already resident in HBM
when timing starts.

The timed steps rotate over enough independent buffer sets (>= 512 MiB, twice
the 256 MiB Infinity Cache) that no step finds its inputs in the
memory-side cache from the previous visit. Steps are replayed from a HIP graph
so host launch overhead does not throttle the GPU; the graph holds exactly the
kernels an eager step launches.

Prints one JSON line. See --help for options.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
METRIC = "dispatch+combine µs & HBM GB/s (% of peak), 128 tok×7168 hidden, 256E top-8"
KERNEL_SOURCES = ("combine_moe_layout_03_amd/csrc/scatter.hip",
                  "combine_moe_layout_03_amd/csrc/fused.hip",
                  "combine_moe_layout_03_amd/csrc/fp8.hpp",
                  "combine_moe_layout_03_amd/csrc/layout.hip",
                  "combine_moe_layout_03_amd/csrc/wave.hpp",
                  "combine_moe_layout_03_amd/csrc/kernels.hpp")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algo_bytes(T, H, K, E, R, P_valid, fp8_flags=None):
    """Bytes the method must move (not what a kernel happens to move). With
    fp8_flags, dispatch writes E4M3 rows (H bytes) plus one 4-byte scale per
    128 channels (one 4-byte UE8M0 word per 512 with MOE_FP8_UE8M0)."""
    row = 2 * H
    dispatch = P_valid * (row + 4) + T * row
    if fp8_flags is not None:
        scale_bytes = 4 * (H // 512 if fp8_flags & 2 else H // 128)
        dispatch = P_valid * (H + scale_bytes + 4) + T * row
    combine = P_valid * (row + 8) + T * row
    layout = T * K * 8 + P_valid * 4 + P_valid * 4 + E * 4 * 2 + 4 + R * 4 + T * R
    return dict(layout=layout, dispatch=dispatch, combine=combine,
                total=layout + dispatch + combine)


def device_hbm_figures(dev_index):
    """Memory bus width and clock as the HIP runtime reports them, and the peak
    they imply for HBM3/HBM3E, which moves four transfers per reported clock
    (bytes/s = 4 x clock x width / 8; the same rule gives MI300X's published
    5.3 TB/s from its 1.3 GHz). The roofline uses the published 8 TB/s; this
    is a cross-check reported beside it."""
    import ctypes
    path = "libamdhip64.so"
    try:  # the HIP runtime torch already loaded, if any
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        hip = ctypes.CDLL(path)
    except OSError:
        return None
    vals = {}
    # hipDeviceAttributeMemoryBusWidth = 59, hipDeviceAttributeMemoryClockRate = 60
    for name, attr in (("bus_width_bits", 59), ("memory_clock_khz", 60)):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev_index) != 0:
            return None
        vals[name] = v.value
    vals["implied_peak_GBps"] = round(4 * vals["memory_clock_khz"] * 1e3
                                      * vals["bus_width_bits"] / 8 / 1e9, 1)
    return vals


def kernel_source_hash():
    """Hash of the measured kernels' code: comments and whitespace are left
    out, so a comment edit does not invalidate the counter summary."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic_c2.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", txt)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"^traffic_bytes_{kernel}:\s*([0-9.]+)", txt, re.M)
    return float(m.group(1)) if m else None


class Workset:
    """One independent set of device buffers for a step."""

    def __init__(self, capi, w, dev):
        import numpy as np
        import torch

        self.shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, w.A)
        self.x = torch.from_numpy(w.x.view(np.int16)).to(dev)
        self.idx = torch.from_numpy(w.topk_idx).to(dev)
        self.w = torch.from_numpy(w.topk_weights).to(dev)
        self.lay = capi.LayoutBuffers.empty(self.shape, dev, status=False)
        self.rows = capi.moe_recv_rows_worst(self.shape)
        self.recv = torch.empty(self.rows, w.H, dtype=torch.int16, device=dev)
        self.out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev)
        n = capi.moe_layout_workspace_bytes(self.shape)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
        self.nbytes = sum(t.numel() * t.element_size() for t in
                          (self.x, self.idx, self.w, self.recv, self.out, self.lay.count,
                           self.lay.offset, self.lay.slot, self.lay.row_src))


def step(capi, s, stream):
    capi.moe_layout_dispatch(s.shape, s.idx, s.lay, s.x, s.recv, s.rows, s.ws, stream=stream)
    capi.moe_combine(s.shape, s.recv, s.rows, s.lay.slot, s.w, s.out, None, None, stream=stream)


def time_graph_steps(torch, graphs_full, graph_rem, reps, stream):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(reps):
            graphs_full.replay()
        if graph_rem is not None:
            graph_rem.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)  # ms


def per_launch_event_times(torch, fn, n, stream):
    """Each launch bracketed by its own pair of events (GPU timestamps)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)  # us
    return dict(mean_us=sum(ts) / n, median_us=ts[n // 2], min_us=ts[0])


def cpu_baseline(w, budget_s, gpu_out_bits):
    """The oracle, as it stands, on this workload's step; single thread."""
    import numpy as np

    import oracle

    orc = oracle.get()
    reps = 0
    t0 = time.perf_counter()
    ref = None
    while True:
        lay = orc.layout(w.topk_idx, w.E, w.R, w.A)
        recv, _ = orc.dispatch(w.x, lay["slot"], lay["rows"])
        ref = orc.combine(recv, lay["slot"], w.topk_weights, "f64")["out_f64"]
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 100000:
            break
    # parity re-check of the timed GPU output against the oracle
    got = (gpu_out_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok = bool(np.all(np.abs(got - ref) <= 1e-3 + 1e-2 * np.abs(ref)))
    return reps, el, ok


def graph_us_per_step(torch, stream, step_fns, reps):
    """Capture one HIP graph holding one step per entry of step_fns, replay it
    `reps` times between events; microseconds per step."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for fn in step_fns:
            fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(reps):
            g.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (reps * len(step_fns))


def row_low_latency(capi, mi, torch, np, dev, stream, fp8_flags=None, M=128):
    """Low-latency padded path at M tokens per rank: layout + dispatch into
    the [E, R*M, H] union of the receive buffers, then combine from it. Steps
    rotate over union buffers x 8 source stripes, enough for > 512 MiB of
    touched bytes (at least 4 unions at M = 128).
    With fp8_flags, dispatch casts to E4M3 + per-128-channel scales
    (moe_ll_layout_dispatch_fp8) and combine reads a bf16 expert-output union
    of the same layout (filled once by a bf16 dispatch of the same batch)."""
    w = mi.config_c3(M)
    E, R, K, T, H = w.E, w.R, w.K, w.T, w.H
    rows = capi.moe_ll_recv_rows(E, R, M)
    shape = capi.make_shape(T, H, E, R, K, 1)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    idx = torch.from_numpy(w.topk_idx).to(dev)
    wt = torch.from_numpy(w.topk_weights).to(dev)
    fp8 = fp8_flags is not None
    P = int((w.topk_idx >= 0).sum())
    ab = algo_bytes(T, H, K, E, R, P, fp8_flags)
    n_unions = max(4 if M == 128 else 1, math.ceil(512 * 2**20 / (ab["total"] * R)))
    unions = [torch.empty(rows, H, dtype=torch.int16, device=dev) for _ in range(n_unions)]
    if fp8:
        cols = capi.fp8_scale_cols(H, fp8_flags)
        sdt = torch.int32 if fp8_flags & capi.MOE_FP8_UE8M0 else torch.float32
        qunions = [torch.empty(rows, H, dtype=torch.uint8, device=dev) for _ in range(n_unions)]
        sshape = (rows, cols) if fp8_flags & capi.MOE_FP8_SCALE_ROWS else (E, cols, R * M)
        sunions = [torch.empty(sshape, dtype=sdt, device=dev) for _ in range(n_unions)]
    sets = []
    for ui, u in enumerate(unions):
        for s in range(R):
            z = dict(u=u, s=s, x=x.clone(), idx=idx.clone(), w=wt.clone(),
                     lay=capi.LayoutBuffers.empty(shape, dev, ll_M=M, status=False,
                                                  rank_tables=False),
                     out=torch.empty(T, H, dtype=torch.int16, device=dev))
            if fp8:
                z.update(q=qunions[ui], sc=sunions[ui])
            sets.append(z)

    def ld(z):
        if fp8:
            capi.moe_ll_layout_dispatch_fp8(shape, M, z["s"], z["idx"], z["lay"], z["x"], z["q"],
                                            z["sc"], rows, fp8_flags, stream=stream)
        else:
            capi.moe_ll_layout_dispatch(shape, M, z["s"], z["idx"], z["lay"], z["x"], z["u"],
                                        rows, stream=stream)

    def cb(z):
        capi.moe_combine(shape, z["u"], rows, z["lay"].slot, z["w"], z["out"], None, None,
                         stream=stream)

    with torch.cuda.stream(stream):
        for z in sets:
            if fp8:  # expert output: the bf16 rows of the same layout
                capi.moe_ll_layout_dispatch(shape, M, z["s"], z["idx"], z["lay"], z["x"], z["u"],
                                            rows, stream=stream)
            ld(z)
            cb(z)
    torch.cuda.synchronize()
    fns = [(lambda z=z: (ld(z), cb(z))) for z in sets]
    us = graph_us_per_step(torch, stream, fns, 20)
    k_ld = graph_us_per_step(torch, stream, [(lambda z=z: ld(z)) for z in sets], 20)
    k_cb = graph_us_per_step(torch, stream, [(lambda z=z: cb(z)) for z in sets], 20)
    n_sets = len(sets)
    del unions, sets
    if fp8:
        del qunions, sunions
    torch.cuda.empty_cache()
    name = "low-latency padded" + (f" FP8 (flags {fp8_flags}: "
                                   + ("row-major" if fp8_flags & 4 else "column-major")
                                   + " scales)" if fp8 else "")
    res = {"workload": name + f": {M} tokens/rank x 7168, 256E top-8, 8 ranks, union receive "
                              f"buffer [256, 8*{M}, 7168]",
           "buffer_sets": n_sets,
           "us_per_step": round(us, 3), "GB_per_s": round(ab["total"] / us / 1e3, 1),
           "kernels_us": {"ll_layout_dispatch" + ("_fp8" if fp8 else ""): round(k_ld, 3),
                          "combine": round(k_cb, 3)},
           "algorithmic_bytes_per_step": ab["total"]}
    res["roofline_dispatch"] = {"achieved": round((ab["layout"] + ab["dispatch"]) / k_ld / 1e3, 1),
                                "frac": round((ab["layout"] + ab["dispatch"]) / k_ld / 1e3
                                              / HBM_PEAK_GBS, 4)}
    return res


def row_normal(capi, mi, torch, np, dev, stream):
    """Normal-mode path on the standard batch (128 tokens x 7168, 256 experts
    top-8 on 8 ranks): one receive row per (token, rank reached), then the
    unweighted row sum and the weight reduce. 30 rotating buffer sets."""
    w = mi.config_c2()
    E, R, K, T, H = w.E, w.R, w.K, w.T, w.H
    shape = capi.make_shape(T, H, E, R, K, 1)
    cap = capi.moe_rank_recv_rows_worst(shape)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    idx = torch.from_numpy(w.topk_idx).to(dev)
    wt = torch.from_numpy(w.topk_weights).to(dev)
    sets = []
    for _ in range(30):
        sets.append(dict(x=x.clone(), idx=idx.clone(), w=wt.clone(),
                         lay=capi.RankLayoutBuffers.empty(shape, dev),
                         recv=torch.empty(cap, H, dtype=torch.int16, device=dev),
                         out=torch.empty(T, H, dtype=torch.int16, device=dev),
                         ow=torch.empty(T, K, dtype=torch.float32, device=dev)))

    def lay(z):
        capi.moe_rank_layout(shape, z["idx"], z["w"], z["lay"], stream=stream)

    def dsp(z):
        capi.moe_rank_dispatch(shape, z["x"], z["lay"].rank_slot, z["recv"], cap, None,
                               stream=stream)

    def lay_dsp(z):
        capi.moe_rank_layout_dispatch(shape, z["idx"], z["w"], z["lay"], z["x"], z["recv"], cap,
                                      stream=stream)

    def cmb(z):
        capi.moe_rank_combine(shape, z["recv"], cap, z["lay"].rank_slot,
                              z["lay"].recv_topk_weights, z["out"], None, z["ow"], None,
                              stream=stream)

    with torch.cuda.stream(stream):
        for z in sets:
            lay(z)
            dsp(z)
            lay_dsp(z)
            cmb(z)
    torch.cuda.synchronize()
    rows = int(sets[0]["lay"].rank_offset[R].item())
    us = graph_us_per_step(torch, stream, [(lambda z=z: (lay_dsp(z), cmb(z))) for z in sets], 20)
    us_two = graph_us_per_step(torch, stream,
                               [(lambda z=z: (lay(z), dsp(z), cmb(z))) for z in sets], 20)
    k = {n: graph_us_per_step(torch, stream, [(lambda z=z, f=f: f(z)) for z in sets], 20)
         for n, f in (("rank_layout_dispatch", lay_dsp), ("rank_combine", cmb),
                      ("rank_layout", lay), ("rank_dispatch", dsp))}
    b_layout = T * K * 12 + T * R * 4 + (R + 1) * 4 + rows * (4 + K * 12) + E * 4
    b_dispatch = T * 2 * H + rows * 2 * H
    b_combine = rows * 2 * H + T * 2 * H + T * R * 4 + rows * K * 4 + T * K * 4
    total = b_layout + b_dispatch + b_combine
    b_fused = b_layout + b_dispatch
    del sets
    torch.cuda.empty_cache()
    return {"workload": "normal mode: 128 tokens x 7168, 256E top-8 on 8 ranks, one row per "
                        "(token, rank): %d rows for %d pairs" % (rows, int((w.topk_idx >= 0).sum())),
            "us_per_step": round(us, 3), "GB_per_s": round(total / us / 1e3, 1),
            "us_per_step_layout_then_dispatch": round(us_two, 3),
            "kernels_us": {n: round(v, 3) for n, v in k.items()},
            "algorithmic_bytes_per_step": total,
            "roofline_layout_dispatch": {
                "achieved": round(b_fused / k["rank_layout_dispatch"] / 1e3, 1),
                "frac": round(b_fused / k["rank_layout_dispatch"] / 1e3 / HBM_PEAK_GBS, 4)}}


def row_replica_train(capi, mi, torch, np, dev, stream):
    """Replica weight sync and replica gradient reduction for the replica
    workload's plan (256 logical experts, 32 replicas on 8 ranks), with one
    7168 x 2048 matrix per expert (a stand-in: the pages give no expert size):
    bf16 weights, f32 gradients, 288 physical experts."""
    w5 = mi.config_c5(T=8192, H=8)
    E, R, C = w5.E, w5.R, w5.replicas
    Ep = E + C
    S = 7168 * 2048
    i32 = dict(dtype=torch.int32, device=dev)
    idx = torch.from_numpy(w5.topk_idx).to(dev)
    load = torch.empty(E, **i32)
    rc = torch.empty(E, **i32)
    rp = torch.empty(E, 2, **i32)
    p2l = torch.empty(Ep, **i32)
    capi.moe_expert_load(w5.T, w5.K, E, idx, load)
    capi.moe_plan_replicas(E, R, C, load, rc, rp, p2l)
    w = torch.zeros(Ep * S, dtype=torch.int16, device=dev)
    g = torch.zeros(Ep * S, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def timed(fn, n=5):
        with torch.cuda.stream(stream):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    t_sync = timed(lambda: capi.moe_replica_weight_sync(E, Ep, S, rc, rp, w, stream=stream))
    t_red = timed(lambda: capi.moe_replica_grad_reduce(E, Ep, S, rc, rp, g, stream=stream))
    b_sync = 2 * C * S * 2
    b_red = 3 * C * S * 4
    del w, g
    torch.cuda.empty_cache()
    return {"workload": "replica weight sync (bf16) and gradient reduction (f32), 256 experts + 32 "
                        "replicas, one 7168x2048 matrix per expert",
            "weight_sync_us": round(t_sync, 1), "grad_reduce_us": round(t_red, 1),
            "weight_sync_GB_per_s": round(b_sync / t_sync / 1e3, 1),
            "grad_reduce_GB_per_s": round(b_red / t_red / 1e3, 1),
            "frac_weight_sync": round(b_sync / t_sync / 1e3 / HBM_PEAK_GBS, 4),
            "frac_grad_reduce": round(b_red / t_red / 1e3 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": {"weight_sync": b_sync, "grad_reduce": b_red}}


def row_config(capi, mi, torch, np, dev, stream, name):
    """The standard step (layout + dispatch in one call, then combine) on
    another configuration: c1 (64 tokens x 256, 16 experts top-2 on 4 ranks)
    or c4 (4096 tokens x 4096, 64 experts top-6 Zipf(1.2) on 8 ranks).
    Rotating buffer sets for >= 512 MiB touched (at most 64 sets)."""
    w = mi.by_name(name)
    probe = Workset(capi, w, dev)
    S = min(64, max(2, math.ceil(512 * 2**20 / probe.nbytes)))
    sets = [probe] + [Workset(capi, w, dev) for _ in range(S - 1)]
    with torch.cuda.stream(stream):
        for z in sets:
            step(capi, z, stream)
    torch.cuda.synchronize()
    us = graph_us_per_step(torch, stream, [(lambda z=z: step(capi, z, stream)) for z in sets],
                           max(4, 200 // S))
    k_ld = graph_us_per_step(torch, stream, [(lambda z=z: capi.moe_layout_dispatch(
        z.shape, z.idx, z.lay, z.x, z.recv, z.rows, z.ws, stream=stream)) for z in sets],
        max(4, 200 // S))
    k_cb = graph_us_per_step(torch, stream, [(lambda z=z: capi.moe_combine(
        z.shape, z.recv, z.rows, z.lay.slot, z.w, z.out, None, None, stream=stream))
        for z in sets], max(4, 200 // S))
    P = int((w.topk_idx >= 0).sum())
    ab = algo_bytes(w.T, w.H, w.K, w.E, w.R, P)
    foot = S * probe.nbytes
    del sets, probe
    torch.cuda.empty_cache()
    r_ld = (ab["layout"] + ab["dispatch"]) / k_ld / 1e3
    r_cb = ab["combine"] / k_cb / 1e3
    return {"workload": f"{w.name}: {w.T} tokens x {w.H}, {w.E} experts top-{w.K} on {w.R} ranks",
            "buffer_sets": S, "footprint_MiB": round(foot / 2**20, 1),
            "us_per_step": round(us, 3), "GB_per_s": round(ab["total"] / us / 1e3, 1),
            "algorithmic_bytes_per_step": ab["total"],
            "kernels_us": {"layout_dispatch": round(k_ld, 3), "combine": round(k_cb, 3)},
            "roofline_layout_dispatch": {"achieved": round(r_ld, 1),
                                         "frac": round(r_ld / HBM_PEAK_GBS, 4)},
            "roofline_combine": {"achieved": round(r_cb, 1), "frac": round(r_cb / HBM_PEAK_GBS, 4)}}


def row_replica(capi, mi, torch, np, dev, stream, n_ev):
    """Replica-expanded routing at full size (8192 tokens x 7168, 256 logical
    experts top-8 Zipf(1.0), 32 extra replicas): load -> plan -> reroute ->
    layout + dispatch over 288 physical experts -> combine. Also the large-batch
    dispatch and combine kernels on their own (their HBM roofline)."""
    w = mi.config_c5()
    E, R, K, T, H, C = w.E, w.R, w.K, w.T, w.H, w.replicas
    Ep = E + C
    shape = capi.make_shape(T, H, Ep, R, K, 1)
    x = torch.from_numpy(w.x.view(np.int16)).to(dev)
    idx = torch.from_numpy(w.topk_idx).to(dev)
    wt = torch.from_numpy(w.topk_weights).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    load = torch.empty(E, **i32)
    rc = torch.empty(E, **i32)
    rp = torch.empty(E, 2, **i32)
    p2l = torch.empty(Ep, **i32)
    phys = torch.empty(T, K, dtype=torch.int64, device=dev)
    lay = capi.LayoutBuffers.empty(shape, dev, status=False)
    rows = capi.moe_recv_rows_worst(shape)
    recv = torch.empty(rows, H, dtype=torch.int16, device=dev)
    out = torch.empty(T, H, dtype=torch.int16, device=dev)
    ws = torch.empty(max(capi.moe_layout_workspace_bytes(shape), 1), dtype=torch.uint8,
                     device=dev)

    def step():
        capi.moe_expert_load(T, K, E, idx, load, None, stream=stream)
        capi.moe_plan_replicas(E, R, C, load, rc, rp, p2l, stream=stream)
        capi.moe_reroute(T, K, E, idx, rc, rp, Ep, phys, None, stream=stream)
        capi.moe_layout_dispatch(shape, phys, lay, x, recv, rows, ws, stream=stream)
        capi.moe_combine(shape, recv, rows, lay.slot, wt, out, None, None, stream=stream)

    with torch.cuda.stream(stream):
        step()
        step()
    torch.cuda.synchronize()
    us = graph_us_per_step(torch, stream, [step], 10)
    with torch.cuda.stream(stream):
        k_d = per_launch_event_times(torch, lambda i: capi.moe_dispatch(
            shape, x, lay.slot, recv, rows, None, stream=stream), n_ev // 4, stream)
        k_c = per_launch_event_times(torch, lambda i: capi.moe_combine(
            shape, recv, rows, lay.slot, wt, out, None, None, stream=stream), n_ev // 4, stream)
    P = T * K
    ab = algo_bytes(T, H, K, Ep, R, P)
    reroute_bytes = P * 8 * 3 + E * 4 * 6 + Ep * 4
    total = ab["total"] + reroute_bytes
    rd = ab["dispatch"] / (k_d["mean_us"] * 1e-6) / 1e9
    rcb = ab["combine"] / (k_c["mean_us"] * 1e-6) / 1e9
    del recv, x, out
    torch.cuda.empty_cache()
    return {"workload": "replica-expanded: 8192 tokens x 7168, 256 logical experts top-8 "
                        "Zipf(1.0) + 32 replicas = 288 physical on 8 ranks",
            "us_per_step": round(us, 2), "GB_per_s": round(total / us / 1e3, 1),
            "algorithmic_bytes_per_step": total,
            "kernels_us": {"dispatch": round(k_d["mean_us"], 2),
                           "combine": round(k_c["mean_us"], 2)},
            "roofline_dispatch": {"achieved": round(rd, 1), "frac": round(rd / HBM_PEAK_GBS, 4)},
            "roofline_combine": {"achieved": round(rcb, 1),
                                 "frac": round(rcb / HBM_PEAK_GBS, 4)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating buffer sets (0: enough for >= 512 MiB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graph")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the low-latency and replica-path measurements")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short fixed run for rocprofv3: warm-up, copy calibration, steps")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU: the logical ranks are "
                          "partitions of one GPU's memory, so --gpus above 1 is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch

    import moe_inputs as mi
    from combine_moe_layout_03_amd import capi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '?')} CUs={props.multi_processor_count}")

    w = mi.config_c2()
    P_valid = int((w.topk_idx >= 0).sum())
    ab = algo_bytes(w.T, w.H, w.K, w.E, w.R, P_valid)
    probe = Workset(capi, w, dev)
    S = args.sets or max(2, math.ceil(512 * 2**20 / probe.nbytes))
    sets = [probe] + [Workset(capi, w, dev) for _ in range(S - 1)]
    log(f"workload {w.name}: {S} buffer sets x {probe.nbytes / 2**20:.1f} MiB")
    stream = torch.cuda.Stream()  # default priority

    # eager warm-up (also runs the one-time device check outside any capture)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(capi, sets[i % S], stream)
    torch.cuda.synchronize()
    ref_out = sets[0].out.clone()

    if args.profile_pass:
        # calibration copy of known size for the PMC counters, then steps
        a = torch.empty(256 * 2**20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                step(capi, sets[i % S], stream)
        torch.cuda.synchronize()
        log(f"profile pass done: 3 x copy of 256 MiB, {args.steps} steps")
        return

    K = args.steps
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for i in range(K):
                step(capi, sets[i % S], stream)
            end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        mode = "eager"
    else:
        g_full = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_full, stream=stream):
            for i in range(S):
                step(capi, sets[i], stream)
        rem = K % S
        g_rem = None
        if rem:
            g_rem = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rem, stream=stream):
                for i in range(rem):
                    step(capi, sets[i], stream)
        # graph warm-up replays, then check they reproduce the eager output
        for _ in range(3):
            g_full.replay()
        torch.cuda.synchronize()
        assert torch.equal(sets[0].out, ref_out), "graph replay differs from eager step"
        ms = time_graph_steps(torch, g_full, g_rem, K // S, stream)
        mode = "hip_graph"
    us_step = ms * 1e3 / K
    value = ab["total"] / (us_step * 1e-6) / 1e9
    log(f"{mode}: {K} steps in {ms:.3f} ms -> {us_step:.2f} us/step, {value:.1f} GB/s")
    # secondary: the same step on one buffer set over and over (caches warm)
    warm_us = None
    if not args.eager:
        warm_us = graph_us_per_step(torch, stream, [(lambda: step(capi, sets[0], stream))] * S,
                                    max(4, 400 // S))
        log(f"warm (one buffer set): {warm_us:.2f} us/step")

    # per-kernel durations: each launch bracketed by events, rotating sets
    n = min(400, max(50, K // 4))

    def ev(fn):
        with torch.cuda.stream(stream):
            return per_launch_event_times(torch, fn, n, stream)

    def z(i):
        return sets[i % S]

    # primary: each kernel alone, one HIP graph of S launches over the rotating
    # sets, events around the replays (the configuration of the timed steps);
    # secondary: every launch bracketed by its own event pair (adds the launch
    # latency of an eager launch)
    fns = {
        "layout_dispatch": lambda i: capi.moe_layout_dispatch(
            z(i).shape, z(i).idx, z(i).lay, z(i).x, z(i).recv, z(i).rows, z(i).ws,
            stream=stream),
        "combine": lambda i: capi.moe_combine(
            z(i).shape, z(i).recv, z(i).rows, z(i).lay.slot, z(i).w, z(i).out, None, None,
            stream=stream),
        # reference: the same work as two separate kernels
        "layout": lambda i: capi.moe_layout(z(i).shape, z(i).idx, z(i).lay, z(i).ws,
                                            stream=stream),
        "dispatch": lambda i: capi.moe_dispatch(z(i).shape, z(i).x, z(i).lay.slot, z(i).recv,
                                                z(i).rows, None, stream=stream),
    }
    kern = {}
    for name, fn in fns.items():
        g_us = graph_us_per_step(torch, stream, [(lambda i=i, fn=fn: fn(i)) for i in range(S)],
                                 max(4, n // S))
        e = ev(fn)
        kern[name] = {"mean_us": g_us, "event_mean_us": e["mean_us"],
                      "event_median_us": e["median_us"]}
    kbytes = {"layout_dispatch": ab["layout"] + ab["dispatch"], "combine": ab["combine"],
              "layout": ab["layout"], "dispatch": ab["dispatch"]}
    dom = max(("layout_dispatch", "combine"), key=lambda k: kern[k]["mean_us"])
    dur = kern[dom]["mean_us"]
    achieved = kbytes[dom] / (dur * 1e-6) / 1e9
    traffic = read_traffic(dom)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": kbytes[dom],
                "duration_us": round(dur, 3)}

    rows = {}
    if not args.no_rows:
        rows["low_latency_m128"] = row_low_latency(capi, mi, torch, np, dev, stream)
        log(f"low-latency row: {rows['low_latency_m128']['us_per_step']} us/step")
        sweep = {}
        for M in (16, 32, 64, 256, 512):
            r = row_low_latency(capi, mi, torch, np, dev, stream, M=M)
            sweep[str(M)] = {k: r[k] for k in ("us_per_step", "GB_per_s", "kernels_us",
                                               "buffer_sets")}
            log(f"low-latency M={M}: {r['us_per_step']} us/step")
        m128 = rows["low_latency_m128"]
        sweep["128"] = {k: m128[k] for k in ("us_per_step", "GB_per_s", "kernels_us",
                                             "buffer_sets")}
        rows["low_latency_sweep"] = {
            "workload": "low-latency padded layout + dispatch + combine, M tokens per rank "
                        "(T = M) x 7168, 256E top-8, 8 ranks",
            "by_M": {k: sweep[k] for k in sorted(sweep, key=int)}}
        rows["low_latency_fp8_m128"] = row_low_latency(capi, mi, torch, np, dev, stream, 0)
        log(f"low-latency FP8 row: {rows['low_latency_fp8_m128']['us_per_step']} us/step")
        rows["low_latency_fp8_rowscales_m128"] = row_low_latency(
            capi, mi, torch, np, dev, stream, capi.MOE_FP8_SCALE_ROWS)
        log(f"low-latency FP8 row-major scales: "
            f"{rows['low_latency_fp8_rowscales_m128']['us_per_step']} us/step")
        rows["normal_mode_128x7168"] = row_normal(capi, mi, torch, np, dev, stream)
        log(f"normal-mode row: {rows['normal_mode_128x7168']['us_per_step']} us/step")
        for cname in ("c1", "c4"):
            rows[f"config_{cname}"] = row_config(capi, mi, torch, np, dev, stream, cname)
            log(f"{cname} row: {rows[f'config_{cname}']['us_per_step']} us/step")
        rows["replica_path_8192"] = row_replica(capi, mi, torch, np, dev, stream, n)
        log(f"replica row: {rows['replica_path_8192']['us_per_step']} us/step")
        rows["replica_train"] = row_replica_train(capi, mi, torch, np, dev, stream)
        log(f"replica sync/reduce row: {rows['replica_train']['weight_sync_us']} / "
            f"{rows['replica_train']['grad_reduce_us']} us")

    torch.cuda.synchronize()
    out_bits = sets[0].out.cpu().numpy().view(np.uint16)
    assert np.array_equal(out_bits, ref_out.cpu().numpy().view(np.uint16))

    cpu = None
    if not args.no_cpu_baseline:
        reps, el, ok = cpu_baseline(w, args.cpu_seconds, out_bits)
        cpu_v = ab["total"] * reps / el / 1e9
        cpu = {"value": round(cpu_v, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} full steps (layout+dispatch+combine f64) of the same "
                         f"128x7168 batch in {el:.1f} s, single thread",
               "us_per_step": round(el / reps * 1e6, 1), "parity_ok": ok}
        log(f"cpu oracle: {reps} steps in {el:.1f}s, parity {'ok' if ok else 'FAILED'}")

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "us_per_step": round(us_step, 3),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "standard: 128 tokens x 7168 hidden bf16, 256 experts on 8 "
                               "logical ranks, top-8 uniform, softmax weights, identity expert",
                   "T": w.T, "H": w.H, "E": w.E, "R": w.R, "K": w.K, "A": w.A,
                   "timing": mode, "buffer_sets": S,
                   "footprint_MiB": round(S * probe.nbytes / 2**20, 1),
                   "algorithmic_bytes_per_step": ab["total"]},
        "us_per_step_warm": round(warm_us, 3) if warm_us is not None else None,
        "hbm_peak_reported_by_device": device_hbm_figures(dev.index or 0),
        "kernels_us": {k: round(v["mean_us"], 3) for k, v in kern.items()},
        "kernels_eager_event_us": {k: round(v["event_mean_us"], 3) for k, v in kern.items()},
        "roofline": roofline,
        "rows": rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
