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
memory-side cache from the previous visit. Before every timed region a spin
kernel keeps the GPU busy while the host queues the region's launches, so the
region starts on a full queue whatever the step count: the headline's steps
are the library's calls issued onto the stream (up to 1000 steps; beyond, one
HIP graph of all of them), each call alone is timed as a HIP graph of a few
hundred calls. A graph launch costs the GPU about 6 us of its own, so no
region is made of many short graphs.

Modes:
  (default)            time the steps, print one JSON line
  --profile-pass P     graph replays only, for rocprofv3 (P: standard | all):
                       segments separated by marker launches, listed in
                       --segments-out
  --summarize DIR...   turn rocprofv3 CSV output (kernel trace, or counter
                       passes) into the markdown summaries kept in profiles/
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import re
import statistics
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
METRIC = "dispatch+combine µs & HBM GB/s (% of peak), 128 tok×7168 hidden, 256E top-8"
CSRC = os.path.join(ROOT, "combine_moe_layout_03_amd", "csrc")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "kernel_trace_standard_128x7168.md")
TRACE_ROWS_SUMMARY = os.path.join(ROOT, "profiles", "kernel_trace_rows.md")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic.md")
MARKER = (1, 1)  # marker launch between profile segments: 1 workgroup of 1 thread


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
    """Hash of every kernel source (comments and whitespace left out, so a
    comment edit does not invalidate the committed profile summaries)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                       glob.glob(os.path.join(CSRC, "*.hpp"))):
        with open(path) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(os.path.basename(path).encode())
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def read_summary(path):
    """Machine-read lines `key: value` of a committed profile summary, or {}
    if it is absent or was taken on other kernel sources."""
    if not os.path.exists(path):
        return {}
    txt = open(path).read()
    m = re.search(r"^kernel_source_hash:\s*([0-9a-f]+)", txt, re.M)
    if not m or m.group(1) != kernel_source_hash():
        return {}
    vals = {}
    for m in re.finditer(r"^(trace_us|fetch_kib|write_kib)\s+(.+?):\s*([-0-9.eE]+)\s*$",
                         txt, re.M):
        vals[(m.group(1), m.group(2))] = float(m.group(3))
    return vals


# --------------------------------------------------------------------------
# timing


class Gate:
    """A spin kernel ahead of a timed region: the GPU stays busy while the
    host queues the region's launches, so the start event is followed by a
    full queue (a 20-step region otherwise carries the graph launch's host
    latency). torch.cuda._sleep spins for a number of GPU clock ticks; the
    tick rate is measured once."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(1000)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            torch.cuda._sleep(2_000_000)
            b.record(stream)
        torch.cuda.synchronize()
        self.ticks_per_us = 2_000_000 / max(a.elapsed_time(b) * 1e3, 1.0)

    def hold(self, us):
        self.torch.cuda._sleep(int(us * self.ticks_per_us))


class HipEvent:
    """A timing event created with hipEventDisableSystemFence: recording it
    takes a GPU timestamp without the system-scope cache writeback and
    invalidation a default event performs, which would otherwise be charged
    to the region it closes (a fixed cost per region, 6% of a 20-step run)."""

    _hip = None

    def __init__(self):
        import ctypes as C
        if HipEvent._hip is None:
            h = hip_runtime()
            h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
            h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
            h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
            h.hipEventDestroy.argtypes = [C.c_void_p]
            HipEvent._hip = h
        self.ev = C.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(C.byref(self.ev), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        import ctypes as C
        rc = HipEvent._hip.hipEventRecord(self.ev, C.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes as C
        ms = C.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(C.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        h = getattr(HipEvent, "_hip", None) if HipEvent is not None else None
        if h is not None and self.ev:
            h.hipEventDestroy(self.ev)
            self.ev = None


def timed_ms(torch, stream, gate, enqueue, launches, warm=None, hold_us=None):
    """Events around enqueue() on `stream`, with the device synchronised
    before and after. Ahead of the start event: a spin long enough for the
    host to queue the region (hold_us, else 5 us per graph launch of
    `launches` kernels, 0.2-50 ms), then warm(), untimed work of the same
    kind (so the region starts in the steady state of a long run, not on a
    GPU that idled in the spin)."""
    torch.cuda.synchronize()
    start, end = HipEvent(), HipEvent()
    with torch.cuda.stream(stream):
        gate.hold(hold_us if hold_us is not None else min(50_000, max(200, 5 * launches)))
        if warm is not None:
            warm()
        start.record(stream)
        enqueue()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def hip_runtime():
    """The HIP runtime library torch has loaded (ctypes)."""
    import ctypes
    path = "libamdhip64.so"
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    return ctypes.CDLL(path)


class HipGraph:
    """A HIP graph captured from `stream` with the runtime's own calls (no
    torch graph wrapper: its replay launches two RNG-state fills before the
    graph, which would land in the timed region)."""

    _hip = None

    def __init__(self, stream, fns):
        import ctypes as C
        if HipGraph._hip is None:
            h = hip_runtime()
            h.hipStreamBeginCapture.argtypes = [C.c_void_p, C.c_int]
            h.hipStreamEndCapture.argtypes = [C.c_void_p, C.POINTER(C.c_void_p)]
            h.hipGraphInstantiate.argtypes = [C.POINTER(C.c_void_p), C.c_void_p, C.c_void_p,
                                              C.c_char_p, C.c_size_t]
            h.hipGraphLaunch.argtypes = [C.c_void_p, C.c_void_p]
            h.hipGraphExecDestroy.argtypes = [C.c_void_p]
            h.hipGraphDestroy.argtypes = [C.c_void_p]
            HipGraph._hip = h
        h = HipGraph._hip
        self.s = C.c_void_p(stream.cuda_stream)
        self.graph, self.exec = C.c_void_p(), C.c_void_p()
        self._check(h.hipStreamBeginCapture(self.s, 2), "hipStreamBeginCapture")  # relaxed
        try:
            for fn in fns:
                fn()
        finally:
            rc = h.hipStreamEndCapture(self.s, C.byref(self.graph))
        self._check(rc, "hipStreamEndCapture")
        self._check(h.hipGraphInstantiate(C.byref(self.exec), self.graph, None, None, 0),
                    "hipGraphInstantiate")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")

    def replay(self):
        self._check(HipGraph._hip.hipGraphLaunch(self.exec, self.s), "hipGraphLaunch")

    def __del__(self):
        h = getattr(HipGraph, "_hip", None) if HipGraph is not None else None
        if h is not None and self.exec:
            h.hipGraphExecDestroy(self.exec)
            h.hipGraphDestroy(self.graph)
            self.exec = None


def capture(torch, stream, fns):
    torch.cuda.synchronize()
    return HipGraph(stream, fns)


# Calls per captured graph in graph_us: a graph launch costs the GPU about
# 6 us of its own (the runtime's packets around the graph: a region of N
# standard steps measured 9.5 + 8.73 N us as one graph, 3.2 + 14.8 N us as one
# graph per step), so each graph holds a few hundred calls.
GRAPH_CALLS = 600
# Headline regions up to this many steps are timed as stream launches.
EAGER_STEPS = 1000


def graph_us(torch, stream, gate, fns, reps, launches=1):
    """fns (one call each) captured m times over into one HIP graph (m <=
    reps, about GRAPH_CALLS calls), replayed until about reps rounds of fns
    are done, between events; microseconds per call."""
    m = max(1, min(reps, math.ceil(GRAPH_CALLS / len(fns))))
    n = max(1, round(reps / m))
    g = capture(torch, stream, list(fns) * m)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()

    def go():
        for _ in range(n):
            g.replay()
    ms = timed_ms(torch, stream, gate, go, n * len(fns) * launches, warm=go)
    del g
    return ms * 1e3 / (n * m * len(fns))


# --------------------------------------------------------------------------
# workloads ("rows"): per-set callables for one step and for each API call


class Row:
    """One measured configuration. step: per-set callables of one step;
    calls: name -> per-set callables of one API call each; nbytes: name (and
    "step") -> algorithmic bytes per call; main: the calls a step is made of
    (the roofline takes the longest)."""

    def __init__(self, key, workload, step, calls, nbytes, main, launches=2, reps=None,
                 extra=None, holder=None):
        self.key, self.workload = key, workload
        self.step, self.calls, self.nbytes, self.main = step, calls, nbytes, main
        self.launches = launches  # kernel launches per step
        self.reps = reps
        self.extra = extra or {}
        self.holder = holder  # keeps the buffers alive

    def release(self, torch):
        self.step = self.calls = self.holder = None
        torch.cuda.empty_cache()


def n_sets(set_bytes, min_sets=2, max_sets=64):
    return min(max_sets, max(min_sets, math.ceil(512 * 2**20 / set_bytes)))


class Arena:
    """Device buffers carved from one allocation (256-byte aligned pieces),
    for comparing against one allocation per buffer."""

    def __init__(self, torch, dev, nbytes):
        self.torch = torch
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.off = 0

    def empty(self, *shape, dtype):
        n = math.prod(shape) * self.torch.empty((), dtype=dtype).element_size()
        if self.off + n > self.buf.numel():
            raise MemoryError("arena exhausted")
        t = self.buf[self.off:self.off + n].view(dtype).view(*shape)
        self.off += (n + 255) // 256 * 256
        return t


class Workset:
    """One independent set of device buffers for a step of the standard kind
    (layout + dispatch in one call, combine); from `arena` when given."""

    def __init__(self, capi, w, dev, arena=None):
        import numpy as np
        import torch

        def alloc(*shape, dtype):
            if arena is None:
                return torch.empty(*shape, dtype=dtype, device=dev)
            return arena.empty(*shape, dtype=dtype)

        def upload(a, dtype):
            t = alloc(*a.shape, dtype=dtype)
            t.copy_(torch.from_numpy(a))
            return t

        self.shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, w.A)
        self.x = upload(w.x.view(np.int16), torch.int16)
        self.idx = upload(w.topk_idx, torch.int64)
        self.w = upload(w.topk_weights, torch.float32)
        T, E, R, K = w.T, w.E, w.R, w.K
        self.rows = capi.moe_recv_rows_worst(self.shape)
        self.lay = capi.LayoutBuffers(
            count=alloc(E, dtype=torch.int32), offset=alloc(E + 1, dtype=torch.int32),
            slot=alloc(T * K, dtype=torch.int32), rank_token_count=alloc(R, dtype=torch.int32),
            is_token_in_rank=alloc(T * R, dtype=torch.uint8),
            row_src=alloc(max(self.rows, 1), dtype=torch.int32))
        self.recv = alloc(self.rows, w.H, dtype=torch.int16)
        self.out = alloc(w.T, w.H, dtype=torch.int16)
        n = capi.moe_layout_workspace_bytes(self.shape)
        self.ws = alloc(n, dtype=torch.uint8) if n else None
        self.nbytes = sum(t.numel() * t.element_size() for t in
                          (self.x, self.idx, self.w, self.recv, self.out, self.lay.count,
                           self.lay.offset, self.lay.slot, self.lay.row_src))


def workset_bytes(w, ws_bytes):
    """Device bytes of one Workset of workload w (each piece rounded up to 256
    as the arena places them); ws_bytes: its layout workspace."""
    r = lambda n: (n + 255) // 256 * 256  # noqa: E731
    T, H, E, R, K = w.T, w.H, w.E, w.R, w.K
    rows = T * K + E * (w.A - 1)
    return (r(T * H * 2) + r(T * K * 8) + r(T * K * 4) + r(E * 4) + r((E + 1) * 4)
            + r(T * K * 4) + r(R * 4) + r(T * R) + r(max(rows, 1) * 4) + r(rows * H * 2)
            + r(T * H * 2) + r(ws_bytes))


def standard_calls(capi, z, stream):
    return {
        "layout_dispatch": lambda: capi.moe_layout_dispatch(
            z.shape, z.idx, z.lay, z.x, z.recv, z.rows, z.ws, stream=stream),
        "combine": lambda: capi.moe_combine(
            z.shape, z.recv, z.rows, z.lay.slot, z.w, z.out, None, None, stream=stream),
        # reference: the same work as two separate kernels
        "layout": lambda: capi.moe_layout(z.shape, z.idx, z.lay, z.ws, stream=stream),
        "dispatch": lambda: capi.moe_dispatch(z.shape, z.x, z.lay.slot, z.recv, z.rows, None,
                                              stream=stream),
    }


def row_standard_kind(capi, mi, torch, dev, stream, name, key, sets=0, arena=False):
    """The standard step (layout + dispatch in one call, then combine) on a
    workload: c2 (the headline), c1 or c4; rotating sets for >= 512 MiB.
    arena: every set carved from one allocation."""
    w = mi.by_name(name)
    nws = capi.moe_layout_workspace_bytes(capi.make_shape(w.T, w.H, w.E, w.R, w.K, w.A))
    per_set = workset_bytes(w, nws)
    S = sets or n_sets(per_set)
    ar = Arena(torch, dev, S * per_set) if arena else None
    zs = [Workset(capi, w, dev, ar) for _ in range(S)]
    probe = zs[0]
    with torch.cuda.stream(stream):
        for z in zs:
            c = standard_calls(capi, z, stream)
            c["layout_dispatch"]()
            c["combine"]()
    torch.cuda.synchronize()
    calls = {k: [standard_calls(capi, z, stream)[k] for z in zs]
             for k in ("layout_dispatch", "combine", "layout", "dispatch")}
    step = [(lambda z=z: (standard_calls(capi, z, stream)["layout_dispatch"](),
                          standard_calls(capi, z, stream)["combine"]())) for z in zs]
    P = int((w.topk_idx >= 0).sum())
    ab = algo_bytes(w.T, w.H, w.K, w.E, w.R, P)
    nb = {"layout_dispatch": ab["layout"] + ab["dispatch"], "combine": ab["combine"],
          "layout": ab["layout"], "dispatch": ab["dispatch"] + 4 * P, "step": ab["total"]}
    return Row(key, f"{w.name}: {w.T} tokens x {w.H}, {w.E} experts top-{w.K} on {w.R} ranks",
               step, calls, nb, ("layout_dispatch", "combine"),
               extra={"buffer_sets": S, "footprint_MiB": round(S * probe.nbytes / 2**20, 1),
                      "one_allocation": bool(arena), "workload_obj": w}, holder=(zs, ar))


def row_floors(capi, floors, mi, torch, np, dev, stream):
    """Floors at the standard shape (128 tokens x 7168, K = 8): the same bytes
    as the two kernels with nothing data-dependent, and a launch with no work.
    Rotating sets as for the real kernels."""
    T, H, K = 128, 7168, 8
    row = 2 * H
    S = n_sets(T * row * (K + 1) * 2)
    xs = [torch.randn(T, H, device=dev).to(torch.bfloat16).view(torch.int16) for _ in range(S)]
    bc = [torch.empty(T * K, H, dtype=torch.int16, device=dev) for _ in range(S)]
    go = [torch.empty(T, H, dtype=torch.int16, device=dev) for _ in range(S)]
    ncopy = T * row * (K + 1) // 2  # 8.26 MB read + written: the dispatch's 16.5 MB moved
    cs = [torch.empty(ncopy, dtype=torch.uint8, device=dev) for _ in range(S)]
    cd = [torch.empty(ncopy, dtype=torch.uint8, device=dev) for _ in range(S)]
    big_s = torch.empty(256 * 2**20, dtype=torch.uint8, device=dev)
    big_d = torch.empty_like(big_s)
    # a copy four times the 256 MB Infinity Cache each way: the streaming rate
    huge_s = torch.empty(2**30, dtype=torch.uint8, device=dev)
    huge_d = torch.empty_like(huge_s)
    # the same two floors at 512 tokens (the low-latency sweep's largest batch)
    T5 = 512
    S5 = n_sets(T5 * row * (K + 1) * 2)
    xs5 = [torch.randn(T5, H, device=dev).to(torch.bfloat16).view(torch.int16) for _ in range(S5)]
    bc5 = [torch.empty(T5 * K, H, dtype=torch.int16, device=dev) for _ in range(S5)]
    go5 = [torch.empty(T5, H, dtype=torch.int16, device=dev) for _ in range(S5)]
    s = stream
    calls = {
        "empty_1x64": [lambda: floors.empty(1, 64, s)] * S,
        "empty_512x512": [lambda: floors.empty(512, 512, s)] * S,
        "empty_3584x64": [lambda: floors.empty(3584, 64, s)] * S,
        "bcast_128x7168x8": [(lambda i=i: floors.bcast(xs[i], bc[i], T, H, K, s))
                             for i in range(S)],
        "gather_128x7168x8": [(lambda i=i: floors.gather(bc[i], go[i], T, H, K, s))
                              for i in range(S)],
        "bcast2_128x7168x8": [(lambda i=i: floors.bcast_split(xs[i], bc[i], T, H, K, 2, s))
                              for i in range(S)],
        "copy_8.26MB": [(lambda i=i: floors.copy(cs[i], cd[i], ncopy, s)) for i in range(S)],
        "copy_256MiB": [lambda: floors.copy(big_s, big_d, big_s.numel(), s)] * 2,
        "copy_1GiB": [lambda: floors.copy(huge_s, huge_d, huge_s.numel(), s)] * 2,
        "bcast_512x7168x8": [(lambda i=i: floors.bcast(xs5[i], bc5[i], T5, H, K, s))
                             for i in range(S5)],
        "gather_512x7168x8": [(lambda i=i: floors.gather(bc5[i], go5[i], T5, H, K, s))
                              for i in range(S5)],
        "bcast2_512x7168x8": [(lambda i=i: floors.bcast_split(xs5[i], bc5[i], T5, H, K, 2, s))
                              for i in range(S5)],
    }
    with torch.cuda.stream(stream):
        for fns in calls.values():
            for f in fns:
                f()
    torch.cuda.synchronize()
    nb = {"empty_1x64": 0, "empty_512x512": 0, "empty_3584x64": 0,
          "bcast_128x7168x8": T * row * (K + 1), "gather_128x7168x8": T * row * (K + 1),
          "bcast2_128x7168x8": T * row * (K + 1),
          "copy_8.26MB": 2 * ncopy, "copy_256MiB": 2 * big_s.numel(),
          "copy_1GiB": 2 * huge_s.numel(),
          "bcast_512x7168x8": T5 * row * (K + 1), "gather_512x7168x8": T5 * row * (K + 1),
          "bcast2_512x7168x8": T5 * row * (K + 1),
          "step": 0}
    return Row("floors", "floors at 128 tokens x 7168, top-8: empty launches, a broadcast copy "
               "(one row read, 8 sequential row writes per token; also with 2 waves per 1 KiB "
               "chunk, each storing half the rows), a gather + sum (8 row "
               "reads at computed addresses, one row write), plain copies; the broadcast and "
               "the gather also at 512 tokens", None, calls, nb, (),
               extra={"buffer_sets": S, "buffer_sets_512": S5},
               holder=(xs, bc, go, cs, cd, big_s, big_d, huge_s, huge_d, xs5, bc5, go5))


def row_low_latency(capi, mi, torch, np, dev, stream, fp8_flags=None, M=128, masked=False):
    """Low-latency padded path at M tokens per rank: layout + dispatch into
    the [E, R*M, H] union of the receive buffers, then combine from it. Steps
    rotate over union buffers x 8 source stripes, enough for > 512 MiB of
    touched bytes (at least 4 unions from M = 128 on).
    With fp8_flags, dispatch casts to E4M3 + per-128-channel scales
    (moe_ll_layout_dispatch_fp8) and combine reads a bf16 expert-output union
    of the same layout (filled once by a bf16 dispatch of the same batch).
    masked: also the combine with an active-rank mask (no rank masked, and
    rank 3 masked)."""
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
    # at least 4 unions from M = 128 on (the large rows' timings otherwise
    # vary by several percent from one process to the next with where the
    # one union lands in memory)
    n_unions = max(4 if M >= 128 else 1, math.ceil(512 * 2**20 / (ab["total"] * R)))
    unions = [torch.empty(rows, H, dtype=torch.int16, device=dev) for _ in range(n_unions)]
    qunions = sunions = None
    if fp8:
        cols = capi.fp8_scale_cols(H, fp8_flags)
        sdt = torch.int32 if fp8_flags & capi.MOE_FP8_UE8M0 else torch.float32
        qunions = [torch.empty(rows, H, dtype=torch.uint8, device=dev) for _ in range(n_unions)]
        sshape = (rows, cols) if fp8_flags & capi.MOE_FP8_SCALE_ROWS else (E, cols, R * M)
        sunions = [torch.empty(sshape, dtype=sdt, device=dev) for _ in range(n_unions)]
    mask_none = torch.zeros(R, dtype=torch.int32, device=dev)
    mask_one = torch.zeros(R, dtype=torch.int32, device=dev)
    mask_one[3] = 1
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

    def cbm(z, m):
        capi.moe_combine_masked(shape, z["u"], rows, z["lay"].slot, z["idx"], z["w"], m,
                                z["out"], None, None, stream=stream)

    with torch.cuda.stream(stream):
        for z in sets:
            if fp8:  # expert output: the bf16 rows of the same layout
                capi.moe_ll_layout_dispatch(shape, M, z["s"], z["idx"], z["lay"], z["x"], z["u"],
                                            rows, stream=stream)
            ld(z)
            cb(z)
            if masked:
                cbm(z, mask_none)
    torch.cuda.synchronize()
    tag = "ll_layout_dispatch" + ("_fp8" if fp8 else "")
    calls = {tag: [(lambda z=z: ld(z)) for z in sets],
             "combine": [(lambda z=z: cb(z)) for z in sets]}
    nb = {tag: ab["layout"] + ab["dispatch"], "combine": ab["combine"], "step": ab["total"]}
    if masked:
        calls["combine_masked_none"] = [(lambda z=z: cbm(z, mask_none)) for z in sets]
        calls["combine_masked_rank3"] = [(lambda z=z: cbm(z, mask_one)) for z in sets]
        # the ids and the mask are read besides combine's bytes; a masked rank's
        # rows are not summed, but are still read (the row loads do not wait
        # for the mask), so the same bytes move with one rank masked
        nb["combine_masked_none"] = ab["combine"] + 8 * T * K + 4 * R
        nb["combine_masked_rank3"] = ab["combine"] + 8 * T * K + 4 * R
    name = "low-latency padded" + (f" FP8 (flags {fp8_flags}: "
                                   + ("row-major" if fp8_flags & 4 else "column-major")
                                   + " scales)" if fp8 else "")
    key = (f"low_latency_fp8_{'rowscales_' if fp8_flags & 4 else ''}m{M}" if fp8
           else f"low_latency_m{M}")
    return Row(key, name + f": {M} tokens/rank x 7168, 256E top-8, 8 ranks, union receive "
                           f"buffer [256, 8*{M}, 7168]",
               [(lambda z=z: (ld(z), cb(z))) for z in sets], calls, nb, (tag, "combine"),
               extra={"buffer_sets": len(sets)}, holder=(unions, qunions, sunions, sets))


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
    b_layout = T * K * 12 + T * R * 4 + (R + 1) * 4 + rows * (4 + K * 12) + E * 4
    b_dispatch = T * 2 * H + rows * 2 * H
    b_combine = rows * 2 * H + T * 2 * H + T * R * 4 + rows * K * 4 + T * K * 4
    calls = {"rank_layout_dispatch": [(lambda z=z: lay_dsp(z)) for z in sets],
             "rank_combine": [(lambda z=z: cmb(z)) for z in sets],
             "rank_layout": [(lambda z=z: lay(z)) for z in sets],
             "rank_dispatch": [(lambda z=z: dsp(z)) for z in sets]}
    nb = {"rank_layout_dispatch": b_layout + b_dispatch, "rank_combine": b_combine,
          "rank_layout": b_layout, "rank_dispatch": b_dispatch + T * R * 4,
          "step": b_layout + b_dispatch + b_combine}
    return Row("normal_mode_128x7168",
               "normal mode: 128 tokens x 7168, 256E top-8 on 8 ranks, one row per (token, "
               "rank): %d rows for %d pairs" % (rows, int((w.topk_idx >= 0).sum())),
               [(lambda z=z: (lay_dsp(z), cmb(z))) for z in sets], calls, nb,
               ("rank_layout_dispatch", "rank_combine"),
               extra={"buffer_sets": len(sets),
                      "two_launch_step": [(lambda z=z: (lay(z), dsp(z), cmb(z))) for z in sets]},
               holder=sets)


def row_replica(capi, mi, torch, np, dev, stream):
    """Replica-expanded routing at full size (8192 tokens x 7168, 256 logical
    experts top-8 Zipf(1.0), 32 extra replicas): load -> plan -> reroute ->
    layout + dispatch over 288 physical experts -> combine; and the calls on
    their own. One buffer set (2.1 GB per step)."""
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
    s = stream
    fns = {
        "expert_load": lambda: capi.moe_expert_load(T, K, E, idx, load, None, stream=s),
        "plan_replicas": lambda: capi.moe_plan_replicas(E, R, C, load, rc, rp, p2l, stream=s),
        "reroute": lambda: capi.moe_reroute(T, K, E, idx, rc, rp, Ep, phys, None, stream=s),
        "layout": lambda: capi.moe_layout(shape, phys, lay, ws, stream=s),
        "dispatch": lambda: capi.moe_dispatch(shape, x, lay.slot, recv, rows, None, stream=s),
        "combine": lambda: capi.moe_combine(shape, recv, rows, lay.slot, wt, out, None, None,
                                            stream=s),
    }

    def step():
        for k in ("expert_load", "plan_replicas", "reroute", "layout", "dispatch", "combine"):
            fns[k]()

    with torch.cuda.stream(stream):
        step()
        step()
    torch.cuda.synchronize()
    P = T * K
    ab = algo_bytes(T, H, K, Ep, R, P)
    nb = {"expert_load": P * 8 + E * 4, "plan_replicas": E * 4 * 4 + Ep * 4,
          "reroute": P * 8 * 2 + E * 4 * 3, "layout": ab["layout"],
          "dispatch": ab["dispatch"], "combine": ab["combine"]}
    nb["step"] = sum(nb.values())
    calls = {k: [f] for k, f in fns.items()}
    return Row("replica_path_8192",
               "replica-expanded: 8192 tokens x 7168, 256 logical experts top-8 Zipf(1.0) + 32 "
               "replicas = 288 physical on 8 ranks", [step], calls, nb, ("dispatch", "combine"),
               launches=8, reps=10, extra={"buffer_sets": 1},
               holder=(x, idx, wt, load, rc, rp, p2l, phys, lay, recv, out, ws))


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
    wbuf = torch.zeros(Ep * S, dtype=torch.int16, device=dev)
    g = torch.zeros(Ep * S, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    calls = {"weight_sync": [lambda: capi.moe_replica_weight_sync(E, Ep, S, rc, rp, wbuf,
                                                                  stream=stream)],
             "grad_reduce": [lambda: capi.moe_replica_grad_reduce(E, Ep, S, rc, rp, g,
                                                                  stream=stream)]}
    nb = {"weight_sync": 2 * C * S * 2, "grad_reduce": 3 * C * S * 4, "step": 0}
    return Row("replica_train", "replica weight sync (bf16) and gradient reduction (f32), 256 "
               "experts + 32 replicas, one 7168x2048 matrix per expert", None, calls, nb,
               ("weight_sync", "grad_reduce"), reps=5, extra={"buffer_sets": 1},
               holder=(idx, load, rc, rp, p2l, wbuf, g))


# --------------------------------------------------------------------------
# measuring a row


def measure_row(torch, stream, gate, row, reps_hint, pmc, trace):
    """Step time (one graph of a few hundred of the rotating steps) and each
    call alone (likewise); algorithmic GB/s and the fraction of peak;
    HBM bytes from the committed counter summary; the committed trace's
    kernel time per call."""
    res = {"workload": row.workload}
    res.update({k: v for k, v in row.extra.items()
                if k not in ("workload_obj", "two_launch_step")})
    S = len(next(iter(row.calls.values())))
    reps = row.reps or max(4, reps_hint // max(S, 1))
    if row.step:
        us = graph_us(torch, stream, gate, row.step, reps, row.launches)
        res["us_per_step"] = round(us, 3)
        res["GB_per_s"] = round(row.nbytes["step"] / us / 1e3, 1)
        res["algorithmic_bytes_per_step"] = row.nbytes["step"]
    if "two_launch_step" in row.extra:
        us2 = graph_us(torch, stream, gate, row.extra["two_launch_step"], reps, 3)
        res["us_per_step_layout_then_dispatch"] = round(us2, 3)
    kern = {}
    for name, fns in row.calls.items():
        us = graph_us(torch, stream, gate, fns, max(reps, 2) if len(fns) > 1 else reps)
        nb = row.nbytes.get(name, 0)
        d = {"us": round(us, 3), "algorithmic_bytes": nb}
        if nb:
            d["GB_per_s"] = round(nb / us / 1e3, 1)
            d["frac"] = round(nb / us / 1e3 / HBM_PEAK_GBS, 4)
        seg = f"{row.key}/{name}"
        t = pmc.get(("traffic", seg))
        d["traffic"] = round(t) if t is not None else None
        if t is not None and nb:
            d["traffic_ratio"] = round(t / nb, 3)
        tr = trace.get(("trace_us", seg + " per_call"))
        if tr is not None:
            d["trace_us"] = round(tr, 3)
        kern[name] = d
    res["calls"] = kern
    return res


def pmc_traffic(summary):
    """HBM bytes per call of each profiled segment: FETCH_SIZE and WRITE_SIZE
    (KiB per call) scaled by what they read for a copy of known size (the
    floor copy kernel)."""
    out = {}
    f_cal = summary.get(("fetch_kib", "floors/copy_256MiB per_call"))
    w_cal = summary.get(("write_kib", "floors/copy_256MiB per_call"))
    if not f_cal or not w_cal:
        return out
    true_kib = 256 * 1024
    ff, fw = f_cal / true_kib, w_cal / true_kib
    out["factors"] = (ff, fw)
    for (kind, key), v in summary.items():
        if kind != "fetch_kib" or not key.endswith(" per_call"):
            continue
        seg = key[:-len(" per_call")]
        wv = summary.get(("write_kib", key))
        if wv is None:
            continue
        out[("traffic", seg)] = (v / ff + wv / fw) * 1024
    return out


# --------------------------------------------------------------------------
# CPU baseline


def host_cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else affinity
    return model, affinity, threads


def cpu_baseline(w, budget_s, gpu_out_bits, total_bytes):
    """The oracle as it stands on this workload's step, per phase (layout,
    dispatch, float combine): once single-threaded, once on all the host
    cores this process may use (the OpenMP build: dispatch and combine split
    over tokens, the layout pass serial). Each leg's output is checked
    against the timed GPU output (bit for bit against the float path, and
    within 1e-2 / 1e-3 of the double sum)."""
    import numpy as np

    import oracle

    model, affinity, threads = host_cpu_info()
    legs = {}
    ref64 = None
    for leg, orc, nthr in (("single_thread", oracle.get(), 1),
                           ("all_cores", oracle.get_parallel(), threads)):
        used = orc.threads(nthr)
        recv = None
        t = {"layout": [], "dispatch": [], "combine": []}
        t0 = time.perf_counter()
        c = None
        while True:
            a = time.perf_counter()
            lay = orc.layout(w.topk_idx, w.E, w.R, w.A)
            b = time.perf_counter()
            if recv is None or recv.shape[0] < lay["rows"]:
                recv = np.empty((lay["rows"], w.H), np.uint16)
            r, _ = orc.dispatch(w.x, lay["slot"], lay["rows"], out=recv[:lay["rows"]])
            c_ = time.perf_counter()
            c = orc.combine(r, lay["slot"], w.topk_weights, "f32")
            d = time.perf_counter()
            t["layout"].append(b - a)
            t["dispatch"].append(c_ - b)
            t["combine"].append(d - c_)
            if d - t0 >= budget_s / 2 or len(t["layout"]) >= 100000:
                break
        if ref64 is None:
            ref64 = orc.combine(r, lay["slot"], w.topk_weights, "f64")["out_f64"]
        got = (gpu_out_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ok = bool(np.array_equal(c["out_bf16"], gpu_out_bits)) and \
            bool(np.all(np.abs(got - ref64) <= 1e-3 + 1e-2 * np.abs(ref64)))
        n = len(t["layout"])
        step = sum(sum(v) for v in t.values()) / n
        legs[leg] = {"threads": used, "steps": n,
                     "us": {k: round(statistics.median(v) * 1e6, 1) for k, v in t.items()},
                     "us_per_step": round(step * 1e6, 1),
                     "GB_per_s": round(total_bytes / step / 1e9, 3), "parity_ok": ok}
        log(f"cpu oracle {leg} ({used} threads): {n} steps, {step * 1e6:.0f} us/step, "
            f"parity {'ok' if ok else 'FAILED'}")
    a = legs["all_cores"]
    return {"value": a["GB_per_s"], "unit": "GB/s", "cores": a["threads"], "kind": "oracle",
            "sample": f"{a['steps']} full steps (layout, dispatch, float combine) of the "
                      f"standard 128x7168 batch on {a['threads']} threads, and "
                      f"{legs['single_thread']['steps']} on 1 thread, about "
                      f"{budget_s / 2:.0f} s each; per-phase medians in legs",
            "cpu_model": model, "affinity_cores": affinity, "legs": legs,
            "parity_ok": all(v["parity_ok"] for v in legs.values())}


# --------------------------------------------------------------------------
# floor kernels (libmoe_floors.so, measurement only)


class Floors:
    def __init__(self):
        import ctypes as C

        from combine_moe_layout_03_amd import build as hb

        if not os.path.exists(hb.FLOOR_LIB):
            raise ImportError(f"{hb.FLOOR_LIB} is not built; run __graft_entry__.build()")
        self.C = C
        lib = C.CDLL(hb.FLOOR_LIB)
        P, I32, I64 = C.c_void_p, C.c_int32, C.c_int64
        lib.moe_floor_empty.argtypes = [I32, I32, P]
        lib.moe_floor_bcast.argtypes = [P, P, I32, I32, I32, P]
        lib.moe_floor_bcast_split.argtypes = [P, P, I32, I32, I32, I32, P]
        lib.moe_floor_gather.argtypes = [P, P, I32, I32, I32, P]
        lib.moe_floor_copy.argtypes = [P, P, I64, P]
        self.lib = lib

    @staticmethod
    def _s(stream):
        import ctypes as C
        return C.c_void_p(stream.cuda_stream)

    def _ok(self, rc, fn):
        if rc != 0:
            raise RuntimeError(f"{fn} failed ({rc})")

    def empty(self, wgs, threads, stream):
        self._ok(self.lib.moe_floor_empty(wgs, threads, self._s(stream)), "moe_floor_empty")

    def bcast(self, x, out, T, H, K, stream):
        self._ok(self.lib.moe_floor_bcast(x.data_ptr(), out.data_ptr(), T, H, K,
                                          self._s(stream)), "moe_floor_bcast")

    def bcast_split(self, x, out, T, H, K, S, stream):
        self._ok(self.lib.moe_floor_bcast_split(x.data_ptr(), out.data_ptr(), T, H, K, S,
                                                self._s(stream)), "moe_floor_bcast_split")

    def gather(self, y, out, T, H, K, stream):
        self._ok(self.lib.moe_floor_gather(y.data_ptr(), out.data_ptr(), T, H, K,
                                           self._s(stream)), "moe_floor_gather")

    def copy(self, src, dst, nbytes, stream):
        self._ok(self.lib.moe_floor_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                         self._s(stream)), "moe_floor_copy")


# --------------------------------------------------------------------------
# profile pass and summaries


def profile_pass(args, capi, floors, mi, torch, np, dev, stream):
    """Graph replays only: for each segment (a row's step, or one call of a
    row alone), a marker launch, one HIP graph of all the segment's calls
    (reps rounds over the buffer sets), another marker. A kernel trace or a
    counter pass thus sees exactly the timed launches between each pair of
    markers (buffer set-up runs outside them). The segment list goes to
    --segments-out."""
    segs = []
    mark = lambda: floors.empty(MARKER[0], MARKER[1], stream)  # noqa: E731

    def run(seg, fns, calls, reps=1):
        g = capture(torch, stream, list(fns) * reps)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            mark()
            g.replay()
            mark()
        torch.cuda.synchronize()
        del g
        segs.append({"name": seg, "calls": calls * reps})
        log(f"segment {seg}: {calls * reps} calls")

    def do_row(row, step_reps=None, only_step=False):
        # about 100 calls per segment (at least 2 replays), one replay of the
        # largest rows' graphs
        reps = lambda n: step_reps or (1 if row.reps else max(2, math.ceil(100 / n)))  # noqa
        if row.step:
            run(f"{row.key}/step", row.step, len(row.step), reps(len(row.step)))
        if not only_step:
            for name, fns in row.calls.items():
                run(f"{row.key}/{name}", fns, len(fns), reps(len(fns)))
        row.release(torch)

    std = row_standard_kind(capi, mi, torch, dev, stream, "c2", "standard", args.sets,
                            args.arena)
    if args.profile_pass == "standard":
        S = len(std.step)
        do_row(std, step_reps=max(1, args.steps // S), only_step=True)
    else:
        do_row(std)
        do_row(row_floors(capi, floors, mi, torch, np, dev, stream))
        for M in mi.C3_SWEEP:
            do_row(row_low_latency(capi, mi, torch, np, dev, stream, M=M, masked=True))
        for fl in (0, capi.MOE_FP8_SCALE_ROWS):
            do_row(row_low_latency(capi, mi, torch, np, dev, stream, fp8_flags=fl))
        do_row(row_normal(capi, mi, torch, np, dev, stream))
        for name in ("c1", "c4"):
            do_row(row_standard_kind(capi, mi, torch, dev, stream, name, f"config_{name}"))
        do_row(row_replica(capi, mi, torch, np, dev, stream))
        do_row(row_replica_train(capi, mi, torch, np, dev, stream))
    torch.cuda.synchronize()
    os.makedirs(os.path.dirname(os.path.abspath(args.segments_out)), exist_ok=True)
    with open(args.segments_out, "w") as f:
        json.dump({"segments": segs, "kernel_source_hash": kernel_source_hash()}, f, indent=1)
    log(f"profile pass done: {len(segs)} segments -> {args.segments_out}")


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(r, *names):
    for n in names:
        if n in r and r[n] != "":
            return r[n]
    return None


def _short(name):
    """Kernel name without return type, namespaces and argument list."""
    name = name.replace("(anonymous namespace)::", "").strip()
    name = re.sub(r"^void ", "", name)
    name = re.sub(r"^moe::", "", name)
    if name.endswith(")"):  # drop the (balanced) argument list
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    return name.strip()


def _dispatches(d):
    """Dispatches of one rocprofv3 CSV output dir, in dispatch order: name,
    grid and workgroup size (threads), and the duration (kernel trace) or the
    counter values (counter collection; a counter repeated for one dispatch
    is counted once)."""
    disp = {}
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in _csv_rows(path):
            e = disp.setdefault(int(_col(r, "Dispatch_Id", "Correlation_Id")), {})
            e["name"] = _col(r, "Kernel_Name")
            e["grid"] = int(float(_col(r, "Grid_Size_X", "Grid_Size") or 0))
            e["wg"] = int(float(_col(r, "Workgroup_Size_X", "Workgroup_Size") or 0))
            e["dur"] = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in _csv_rows(path):
            e = disp.setdefault(int(_col(r, "Dispatch_Id", "Correlation_Id")), {})
            e["name"] = _col(r, "Kernel_Name")
            e["grid"] = int(float(_col(r, "Grid_Size", "Grid_Size_X") or 0))
            e["wg"] = int(float(_col(r, "Workgroup_Size", "Workgroup_Size_X") or 0))
            e.setdefault("ctr", {}).setdefault(_col(r, "Counter_Name"),
                                               float(_col(r, "Counter_Value")))
    return [disp[i] for i in sorted(disp)]


def _segments(es, names):
    """Split dispatches at the marker launches: segment i lies between marker
    2i and marker 2i + 1 (what runs between segments belongs to none)."""
    marks = [j for j, e in enumerate(es)
             if "floor_empty_kernel" in (e.get("name") or "") and e["grid"] == MARKER[0] * MARKER[1]
             and e["wg"] == MARKER[1]]
    if len(marks) != 2 * len(names):
        raise SystemExit(f"found {len(marks)} markers for {len(names)} segments")
    return {n: es[marks[2 * i] + 1: marks[2 * i + 1]] for i, n in enumerate(names)}


def summarize(dirs, segments_path):
    """Aggregate each segment of rocprofv3 CSV output (a kernel trace, or one
    counter pass per dir): per kernel (name, grid, workgroup) the launches and
    the mean/median/min duration or the mean counter values, and per call of
    the segment the totals. Prints one markdown table (a row per segment and
    kernel) and machine-read `kind segment: value` lines (per call; per
    kernel too where a segment runs several kernels)."""
    seg = json.load(open(segments_path))
    names = [s["name"] for s in seg["segments"]]
    calls = {s["name"]: s["calls"] for s in seg["segments"]}
    per_dir = [_segments(_dispatches(d), names) for d in dirs]
    table, mach = [], []
    cn_all, has_dur = set(), False
    agg = {}
    for sname in names:
        groups = {}  # (kernel, grid, wg) -> {"dur": [...], counter: [...]}
        for segs in per_dir:
            for e in segs[sname]:
                g = groups.setdefault((_short(e["name"]), e["grid"], e["wg"]), {})
                g.setdefault("n", []).append(1)
                if "dur" in e:
                    g.setdefault("dur", []).append(e["dur"])
                    has_dur = True
                for c, v in e.get("ctr", {}).items():
                    g.setdefault(c, []).append(v)
                    cn_all.add(c)
        agg[sname] = groups
    cnames = sorted(cn_all)
    head = ["segment", "calls", "kernel", "grid", "wg", "launches"]
    if has_dur:
        head += ["mean µs", "median µs", "min µs"]
    head += [f"{c} KiB" for c in cnames]
    table.append("| " + " | ".join(head) + " |")
    table.append("|" + "---|" * len(head))
    for sname in names:
        groups = agg[sname]
        tot = {c: 0.0 for c in cnames}
        tot_dur = 0.0
        multi = len(groups) > 1
        for (kn, grid, wg), g in sorted(groups.items(), key=lambda kv: -len(kv[1]["n"])):
            n = len(g.get("dur", [])) or max([len(g.get(c, [])) for c in cnames] or [0])
            cells = [sname, str(calls[sname]), f"`{kn}`", str(grid), str(wg), str(n)]
            if has_dur:
                ds = g.get("dur", [])
                cells += ([f"{statistics.mean(ds):.3f}", f"{statistics.median(ds):.3f}",
                           f"{min(ds):.3f}"] if ds else ["—"] * 3)
                if ds:
                    tot_dur += sum(ds)
                    if multi:
                        mach.append(f"trace_us {sname} {kn}@{grid}: {statistics.mean(ds):.4f}")
            for c in cnames:
                v = g.get(c, [])
                tot[c] += sum(v)
                cells.append(f"{statistics.mean(v):.1f}" if v else "—")
            table.append("| " + " | ".join(cells) + " |")
        if has_dur:
            mach.append(f"trace_us {sname} per_call: {tot_dur / calls[sname]:.4f}")
        for c in cnames:
            kind = {"FETCH_SIZE": "fetch_kib", "WRITE_SIZE": "write_kib"}.get(c, c.lower())
            mach.append(f"{kind} {sname} per_call: {tot[c] / calls[sname]:.2f}")
    print("\n".join(table))
    print("\nMachine-read by bench.py (valid only while the kernel sources hash to the value "
          "below):\n")
    print(f"kernel_source_hash: {seg['kernel_source_hash']}")
    for m in mach:
        print(m)


# --------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating buffer sets (0: enough for >= 512 MiB)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="only the standard step (no floors, other rows)")
    ap.add_argument("--profile-pass", choices=("standard", "all"), default=None,
                    help="graph replays only, for rocprofv3")
    ap.add_argument("--segments-out", default=os.path.join(tempfile.gettempdir(), "moe_segments.json"),
                    help="where --profile-pass writes its segment list (markers between them)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR", default=None,
                    help="rocprofv3 CSV output dirs to summarise (with --segments)")
    ap.add_argument("--segments", default=None)
    ap.add_argument("--only-rows", default=None, metavar="REGEX",
                    help="measure only the rows whose key matches")
    ap.add_argument("--arena", action="store_true",
                    help="carve the standard step's buffer sets from one allocation")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize, args.segments or args.segments_out)
        return

    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be at least 1 and --warmup at least 0"}))
        sys.exit(2)

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
    stream = torch.cuda.Stream()  # default priority
    floors = Floors()

    if args.profile_pass:
        # the library's one-time device check, on a shape whose kernels the
        # timed ones do not share (top-1)
        t1 = capi.make_shape(1, 8, 1, 1, 1, 1)
        lb = capi.LayoutBuffers.empty(t1, dev)
        xx = torch.zeros(1, 8, dtype=torch.int16, device=dev)
        rr = torch.empty(1, 8, dtype=torch.int16, device=dev)
        capi.moe_layout_dispatch(t1, torch.zeros(1, 1, dtype=torch.int64, device=dev), lb, xx,
                                 rr, 1, stream=stream)
        torch.cuda.synchronize()
        profile_pass(args, capi, floors, mi, torch, np, dev, stream)
        return

    gate = Gate(torch, stream)
    pmc = pmc_traffic(read_summary(PMC_SUMMARY))
    trace = {}
    trace.update(read_summary(TRACE_ROWS_SUMMARY))
    trace.update(read_summary(TRACE_SUMMARY))

    # ---- the headline: the standard step, exactly --steps of them ----
    std = row_standard_kind(capi, mi, torch, dev, stream, "c2", "standard", args.sets,
                            args.arena)
    w = std.extra["workload_obj"]
    zs = std.holder[0]
    S = len(zs)
    ab = algo_bytes(w.T, w.H, w.K, w.E, w.R, int((w.topk_idx >= 0).sum()))
    log(f"workload {w.name}: {S} buffer sets, {std.extra['footprint_MiB']} MiB")
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            std.step[i % S]()
    torch.cuda.synchronize()
    ref_out = zs[0].out.clone()
    K = args.steps
    # The K steps cycle over the S buffer sets. Up to EAGER_STEPS steps they
    # are the library's calls issued straight onto the stream, behind a spin
    # that lets the host queue all of them first (a region of N steps so
    # measured 0.9 + 8.89 N us); beyond that, one HIP graph of all K steps
    # (9.5 + 8.73 N us: its launch carries a fixed cost, which a long region
    # amortises). Replaying a graph per buffer set instead added about 6 us
    # per graph launch: 9.3 us per step over 20 steps, 8.99 over 2000.
    if K <= EAGER_STEPS:
        timing = "stream"

        def one_pass():
            for i in range(S):
                std.step[i]()
        # the host's enqueue cost per step, with the GPU held busy meanwhile
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            gate.hold(20_000)
            t0 = time.perf_counter()
            one_pass()
            host_us = (time.perf_counter() - t0) * 1e6 / S
        torch.cuda.synchronize()
        assert torch.equal(zs[0].out, ref_out), "the steps' output changed between passes"

        def go():
            for i in range(K):
                std.step[i % S]()
        ms = timed_ms(torch, stream, gate, go, 2 * K, warm=one_pass,
                      hold_us=min(200_000, 1000 + 3 * host_us * (K + S)))
    else:
        timing = "one_graph"
        g_all = capture(torch, stream, [std.step[i % S] for i in range(K)])
        g_all.replay()
        torch.cuda.synchronize()
        assert torch.equal(zs[0].out, ref_out), "graph replay differs from the eager step"
        ms = timed_ms(torch, stream, gate, g_all.replay, 2 * K, warm=g_all.replay)
        del g_all
    us_step = ms * 1e3 / K
    value = ab["total"] / (us_step * 1e-6) / 1e9
    log(f"step ({timing}): {K} steps in {ms:.3f} ms -> {us_step:.3f} us/step, {value:.1f} GB/s")
    # secondary: the same step on one buffer set over and over (caches warm)
    warm_us = graph_us(torch, stream, gate, [std.step[0]] * S, max(4, 400 // S), 2)
    log(f"warm (one buffer set): {warm_us:.3f} us/step")
    std_res = measure_row(torch, stream, gate, std, 400, pmc, trace)
    out_bits = zs[0].out.cpu().numpy().view(np.uint16)
    assert np.array_equal(out_bits, ref_out.cpu().numpy().view(np.uint16))
    std.release(torch)

    # roofline: the longer of the step's two kernels, live duration from the
    # event-timed graph of that call alone
    kc = std_res["calls"]
    dom = max(std.main, key=lambda k: kc[k]["us"])
    dur = kc[dom]["us"]
    achieved = kc[dom]["algorithmic_bytes"] / (dur * 1e-6) / 1e9
    tr_step = {k[1].split(" ", 1)[1]: v for k, v in trace.items()
               if k[0] == "trace_us" and k[1].startswith("standard/step ")}
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": kc[dom]["traffic"], "algorithmic_bytes": kc[dom]["algorithmic_bytes"],
                "duration_us": dur,
                "trace_mean_us_in_step": {k: round(v, 3) for k, v in tr_step.items()} or None}

    rows = {}
    if not args.no_rows:
        rlist = [lambda: row_floors(capi, floors, mi, torch, np, dev, stream)]
        for M in mi.C3_SWEEP:
            rlist.append(lambda M=M: row_low_latency(capi, mi, torch, np, dev, stream, M=M,
                                                     masked=True))
        for fl in (0, capi.MOE_FP8_SCALE_ROWS):
            rlist.append(lambda fl=fl: row_low_latency(capi, mi, torch, np, dev, stream,
                                                       fp8_flags=fl))
        rlist.append(lambda: row_normal(capi, mi, torch, np, dev, stream))
        for name in ("c1", "c4"):
            rlist.append(lambda name=name: row_standard_kind(capi, mi, torch, dev, stream, name,
                                                             f"config_{name}"))
        rlist.append(lambda: row_replica(capi, mi, torch, np, dev, stream))
        rlist.append(lambda: row_replica_train(capi, mi, torch, np, dev, stream))
        for make in rlist:
            row = make()
            if args.only_rows and not re.search(args.only_rows, row.key):
                row.release(torch)
                continue
            rows[row.key] = measure_row(torch, stream, gate, row, 200, pmc, trace)
            log(f"row {row.key}: " + ", ".join(f"{k} {v['us']} us" for k, v in
                                               rows[row.key]["calls"].items()))
            row.release(torch)
        # the low-latency sweep and the masked combine, side by side
        sweep, masked = {}, {}
        for M in mi.C3_SWEEP:
            if f"low_latency_m{M}" not in rows:
                continue
            r = rows.pop(f"low_latency_m{M}")
            c = r["calls"]
            sweep[str(M)] = {k: r[k] for k in ("us_per_step", "GB_per_s", "buffer_sets")}
            sweep[str(M)]["calls"] = {k: c[k] for k in ("ll_layout_dispatch", "combine")}
            masked[str(M)] = {k: c[k] for k in ("combine", "combine_masked_none",
                                                "combine_masked_rank3")}
            if M == 128:
                rows["low_latency_m128"] = dict(r, calls=sweep["128"]["calls"])
        rows["low_latency_sweep"] = {
            "workload": "low-latency padded layout + dispatch + combine, M tokens per rank "
                        "(T = M) x 7168, 256E top-8, 8 ranks", "by_M": sweep}
        rows["masked_combine"] = {
            "workload": "low-latency combine at M tokens per rank x 7168 (256E top-8, 8 ranks): "
                        "plain, with an active-rank mask of no masked rank, and with rank 3 "
                        "masked (its pairs are left out of the sum)", "by_M": masked}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds, out_bits, ab["total"])

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
                   "timing": timing, "buffer_sets": S,
                   "footprint_MiB": std.extra["footprint_MiB"],
                   "algorithmic_bytes_per_step": ab["total"]},
        "us_per_step_warm": round(warm_us, 3),
        "hbm_peak_reported_by_device": device_hbm_figures(dev.index or 0),
        "kernels_us": {k: v["us"] for k, v in kc.items()},
        "standard_calls": kc,
        "pmc_calibration_factors": list(pmc["factors"]) if "factors" in pmc else None,
        "roofline": roofline,
        "rows": rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
