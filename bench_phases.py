#!/usr/bin/env python3
"""Per-phase timestamps of the fused layout + dispatch kernel and of the
broadcast floor kernel, on the standard workload (128 tokens x 7168 bf16,
256 experts top-8) replayed from a HIP graph over rotating buffer sets; and
of the same kernel in the low-latency layout at 128 tokens per rank, bf16 and
FP8 (row-major and column-major scales).

An instrumented copy of the two kernel sources is built into a temporary
directory (the library's own sources and build are left alone): each wave
reads the GPU's 100 MHz real-time counter at the phase boundaries and stores
the readings with vector stores into a device table, read back after each
replay. The copy differs from the library only by those reads and stores.

Phases (each wave, from its own first instruction): the id loads issued, the
row-chunk load issued, the ids arrived (first barrier), the counting done
(second barrier), the row arrived, (FP8) the cast done, the row stores issued,
the wave's end.

    python3 bench_phases.py            (needs an MI355X; prints a markdown table)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.abspath(__file__))
PKG = "combine_moe_layout_03_amd"

# (anchor in fused.hip, text inserted after it)
FUSED_STAMPS = [
    ("  const int b = blockIdx.x;\n  int st = 0;\n",
     "  unsigned long long ts[10] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0};\n  STAMP(0);\n"),
    ("    if (counting) ids.issue(hidx, P, nthreads, nr);\n", "    STAMP(1);\n"),
    ("      val = __builtin_nontemporal_load(hx + (int64_t)t * hnvec + min(v, hnvec - 1));\n",
     "      STAMP(2);\n"),
    ("    if (counting) ids.settle(P, E, nthreads, pbeg, K, s_tok, st);\n    lds_barrier();\n",
     "    STAMP(3);\n"),
    ("      if (lane < K) atomicAdd(&s_pre[lane], prev);\n    }\n    lds_barrier();\n",
     "    STAMP(4);\n"),
    ("      asm volatile(\"\" : \"+v\"(val));\n      if (kCpw == 2) asm volatile(\"\" : \"+v\"(val2));\n",
     "      STAMP(5);\n"),
    # the FP8 branch: the row arrived, the cast done
    ("    if (kCopy && kFp8 >= 0) {\n      asm volatile(\"\" : \"+v\"(val));\n", "      STAMP(5);\n"),
    ("      const u32x2 codes = {q.lo, q.hi};\n",
     "      asm volatile(\"\" :: \"v\"(codes.x), \"v\"(codes.y), \"v\"(q.scale));\n"
     "      STAMP(8);\n"),
]
FUSED_BEFORE = [("    // 6. this token's handle entries", "    STAMP(6);\n")]
FUSED_END = ("  if (st && p.status) atomicOr(p.status, st);\n}",
             "  if (st && p.status) atomicOr(p.status, st);\n  STAMP(7);\n"
             "  if (lane_id() == 0 && b < 4096)\n"
             "    for (int i = 0; i < 10; ++i) g_stamps[b * 16 + (tid >> 6)][i] = ts[i];\n}")
TABLE = ("namespace moe {\nnamespace {\n",
         "namespace moe {\n__device__ unsigned long long g_stamps[4096 * 16][10];\nnamespace {\n"
         "#define STAMP(i) ts[i] = __builtin_amdgcn_s_memrealtime()\n")
FUSED_EXPORT = """
extern "C" __attribute__((visibility("default"))) int moe_debug_stamps(void *dst, size_t bytes) {
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(moe::g_stamps), bytes, 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : -1;
}
"""

FLOOR_OLD = """  const u32x4 val = __builtin_nontemporal_load(x + (int64_t)t * nvec + v);
  u32x4 *dst = out + (int64_t)t * K * nvec + v;
  for (int k = 0; k < K; ++k) __builtin_nontemporal_store(val, dst + (int64_t)k * nvec);"""
FLOOR_NEW = """  u32x4 val = __builtin_nontemporal_load(x + (int64_t)t * nvec + v);
  ts[2] = __builtin_amdgcn_s_memrealtime();
  asm volatile("" : "+v"(val));
  ts[5] = __builtin_amdgcn_s_memrealtime();
  u32x4 *dst = out + (int64_t)t * K * nvec + v;
  for (int k = 0; k < K; ++k) __builtin_nontemporal_store(val, dst + (int64_t)k * nvec);
  ts[6] = ts[7] = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0 && wid < 4096 * 16)
    for (int i = 0; i < 8; ++i) g_fstamps[wid][i] = ts[i];"""
FLOOR_START_OLD = """  const int wid = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
"""
FLOOR_START_NEW = """  unsigned long long ts[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  ts[0] = __builtin_amdgcn_s_memrealtime();
  const int wid = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
"""
FLOOR_TABLE = ("namespace {\n\ntypedef uint32_t u32x4",
               "__device__ unsigned long long g_fstamps[4096 * 16][8];\nnamespace {\n\n"
               "typedef uint32_t u32x4")
FLOOR_EXPORT = """
extern "C" __attribute__((visibility("default"))) int moe_debug_fstamps(void *dst, size_t bytes) {
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_fstamps), bytes, 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : -1;
}
"""


def _insert(src, anchor, text, before=False):
    if src.count(anchor) != 1:
        raise SystemExit(f"instrumentation anchor not found once: {anchor[:60]!r}")
    return src.replace(anchor, text + anchor if before else anchor + text)


def instrument(dst):
    """Copy the package, moe_inputs and bench.py to dst and add the stamps."""
    for item in (PKG, "moe_inputs", "include", "bench.py"):
        s = os.path.join(ROOT, item)
        d = os.path.join(dst, item)
        if os.path.isdir(s):
            shutil.copytree(s, d, ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.tmp"))
        else:
            shutil.copy(s, d)
    fpath = os.path.join(dst, PKG, "csrc", "fused.hip")
    src = open(fpath).read()
    if src.count(TABLE[0]) != 1:
        raise SystemExit("instrumentation anchor (namespace) not found once")
    src = src.replace(TABLE[0], TABLE[1])
    for anchor, text in FUSED_STAMPS:
        src = _insert(src, anchor, text)
    for anchor, text in FUSED_BEFORE:
        src = _insert(src, anchor, text, before=True)
    if src.count(FUSED_END[0]) != 1:
        raise SystemExit("instrumentation anchor (kernel end) not found once")
    src = src.replace(FUSED_END[0], FUSED_END[1]) + FUSED_EXPORT
    open(fpath, "w").write(src)
    fl = os.path.join(dst, PKG, "csrc", "floors.hip")
    src = open(fl).read()
    for old, new in ((FLOOR_OLD, FLOOR_NEW), (FLOOR_START_OLD, FLOOR_START_NEW), FLOOR_TABLE):
        if src.count(old) != 1:
            raise SystemExit(f"floor instrumentation anchor not found once: {old[:60]!r}")
        src = src.replace(old, new)
    open(fl, "w").write(src + FLOOR_EXPORT)


CHILD = r'''
import ctypes as C, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import bench, moe_inputs as mi
from combine_moe_layout_03_amd import capi, build as hb
assert capi.LIB_PATH.startswith(sys.argv[1])
dev = torch.device("cuda:0"); torch.cuda.set_device(dev)
stream = torch.cuda.Stream()
lib = C.CDLL(capi.LIB_PATH); lib.moe_debug_stamps.argtypes = [C.c_void_p, C.c_size_t]
flib = C.CDLL(hb.FLOOR_LIB); flib.moe_debug_fstamps.argtypes = [C.c_void_p, C.c_size_t]
REPS = 10

def pct(a):
    a = np.sort(np.asarray(a, float)); n = len(a)
    return " | ".join(f"{a[int(n * p)] * 0.01:.2f}" for p in (0.1, 0.5, 0.9))

def table(title, reps, waves, wgs, names):
    print(f"\n### {title}\n")
    print("| phase (us from the wave's start) | p10 | p50 | p90 |")
    print("|---|---|---|---|")
    for i, nm in names:
        v = [int(r[b * 16 + w][i]) - int(r[b * 16 + w][0]) if waves > 1 else int(r[b][i]) - int(r[b][0])
             for r in reps for b in range(wgs) for w in range(waves)
             if (r[b * 16 + w] if waves > 1 else r[b])[0]]
        print(f"| {nm} | {pct(v)} |")
    st, en = [], []
    for r in reps:
        rows = [r[b * 16 + w] if waves > 1 else r[b] for b in range(wgs) for w in range(waves)]
        t0 = min(int(x[0]) for x in rows if x[0])
        st += [int(x[0]) - t0 for x in rows if x[0]]
        en += [int(x[7]) - t0 for x in rows if x[7]]
    print(f"| wave start, from the launch's first wave | {pct(st)} |")
    print(f"| wave end, from the launch's first wave | {pct(en)} |")

std = bench.row_standard_kind(capi, mi, torch, dev, stream, "c2", "standard")
S = len(std.step)
g = bench.capture(torch, stream, std.step)
for _ in range(20):
    g.replay()
torch.cuda.synchronize()
buf = np.zeros((4096 * 16, 10), np.uint64)
fbuf = np.zeros((4096 * 16, 8), np.uint64)
reps = []
for _ in range(REPS):
    g.replay(); torch.cuda.synchronize()
    assert lib.moe_debug_stamps(buf.ctypes.data, buf.nbytes) == 0
    reps.append(buf[:512 * 16].copy())
table(f"fused layout + dispatch (standard step graph, {S} buffer sets; the last step's kernel "
      f"of {REPS} replays): 256 token workgroups x 8 waves", reps, 8, 256,
      [(1, "id loads issued"), (2, "row load issued"), (3, "ids in (first barrier)"),
       (4, "counted (second barrier)"), (5, "row in"), (6, "row stores issued"), (7, "end")])
del g
std.release(torch)
T, H, K = 128, 7168, 8
fl = bench.Floors()
xs = [torch.randn(T, H, device=dev).to(torch.bfloat16).view(torch.int16) for _ in range(S)]
bc = [torch.empty(T * K, H, dtype=torch.int16, device=dev) for _ in range(S)]
g2 = bench.capture(torch, stream, [(lambda i=i: fl.bcast(xs[i], bc[i], T, H, K, stream))
                                   for i in range(S)])
for _ in range(20):
    g2.replay()
torch.cuda.synchronize()
reps = []
for _ in range(REPS):
    g2.replay(); torch.cuda.synchronize()
    assert flib.moe_debug_fstamps(fbuf.ctypes.data, fbuf.nbytes) == 0
    reps.append(fbuf[:1792].copy())
table("broadcast floor (same bytes, computed destinations): 1792 waves", reps, 1, 1792,
      [(2, "row load issued"), (5, "row in"), (6, "row stores issued"), (7, "end")])
del g2, xs, bc
torch.cuda.empty_cache()

# the low-latency layout at 128 tokens per rank: bf16, FP8 with row-major and
# with column-major (the page's format) scales
common = [(1, "id loads issued"), (2, "row load issued"), (3, "ids in (first barrier)"),
          (4, "counted (second barrier)"), (5, "row in")]
for flags, name, call in ((None, "bf16", "ll_layout_dispatch"),
                          (4, "FP8, row-major scales", "ll_layout_dispatch_fp8"),
                          (0, "FP8, column-major scales", "ll_layout_dispatch_fp8")):
    row = bench.row_low_latency(capi, mi, torch, np, dev, stream, fp8_flags=flags, M=128)
    g3 = bench.capture(torch, stream, row.calls[call])
    for _ in range(20):
        g3.replay()
    torch.cuda.synchronize()
    reps = []
    for _ in range(REPS):
        g3.replay(); torch.cuda.synchronize()
        assert lib.moe_debug_stamps(buf.ctypes.data, buf.nbytes) == 0
        reps.append(buf[:256 * 16].copy())
    extra = [] if flags is None else [(8, "cast done")]
    table(f"low-latency layout + dispatch, 128 tokens per rank, {name} (graph of "
          f"{len(row.calls[call])} calls over rotating receive unions; the last call's kernel of "
          f"{REPS} replays): 256 token workgroups x 8 waves", reps, 8, 256,
          common + extra + [(6, "row stores issued"), (7, "end")])
    del g3
    row.release(torch)
    del row
    torch.cuda.empty_cache()
'''


def main():
    with tempfile.TemporaryDirectory(prefix="moe_phases_") as tmp:
        instrument(tmp)
        sys.path.insert(0, tmp)
        import importlib
        b = importlib.import_module(f"{PKG}.build")
        if not b.PKG.startswith(tmp):
            raise SystemExit("instrumented build would overwrite the library")
        b.build()
        print("# Per-phase timestamps, standard and low-latency workloads (128 tokens x 7168, "
              "256 experts top-8)\n")
        print("Instrumented copy of the kernels (bench_phases.py): each wave reads the GPU's "
              "100 MHz\nreal-time counter at the phase boundaries; 10 replays, the last step's "
              "kernel of each.\n\n    python3 bench_phases.py    (repository root, one MI355X)")
        sys.stdout.flush()
        r = subprocess.run([sys.executable, "-c", CHILD, tmp])
        sys.exit(r.returncode)


if __name__ == "__main__":
    main()
