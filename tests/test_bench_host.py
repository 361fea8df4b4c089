"""Host logic of bench.py on the CPU: the rocprofv3 summary (segments split at
the marker launches, per-call totals), the reader of committed summaries and
the counter scaling, on synthetic CSV files shaped like rocprofv3's output."""
import csv
import io
import json
import os
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp",
              "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X",
              "Grid_Size_Y", "Grid_Size_Z"]
PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]
MARK = ("floor_empty_kernel()", 1, 1)


def _dispatch_list():
    """(kernel, grid, workgroup, ns duration) in launch order: a warm-up call,
    then segments a (2 calls of two kernels) and b (3 calls of one)."""
    k1 = ("moe::(anonymous namespace)::count_layout_kernel<true, 2, -1>(CountParams)", 262144, 512)
    k2 = ("combine_kernel<8, true>(void const*)", 229376, 64)
    return ([(("warm", 8, 8), 100), (MARK, 10)] + [(k1, 4000), (k2, 5000)] * 2
            + [(MARK, 10), (("setup", 8, 8), 100), (MARK, 10)] + [(k2, 3000)] * 3 + [(MARK, 10)]
            + [(("after", 8, 8), 100)])


def _write_trace(d):
    os.makedirs(os.path.join(d, "host", "123"))
    with open(os.path.join(d, "host", "123", "run_kernel_trace.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, TRACE_COLS)
        wr.writeheader()
        t = 1000
        for i, ((name, grid, wg), dur) in enumerate(_dispatch_list()):
            wr.writerow({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i + 1, "Kernel_Name": name,
                         "Correlation_Id": i + 1, "Start_Timestamp": t, "End_Timestamp": t + dur,
                         "Workgroup_Size_X": wg, "Grid_Size_X": grid})
            t += dur + 50


def _write_pmc(d, counter, per_kernel):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, PMC_COLS)
        wr.writeheader()
        for i, ((name, grid, wg), _) in enumerate(_dispatch_list()):
            v = next((val for key, val in per_kernel.items() if key in name), 0.0)
            for _ in range(2):  # a counter repeated for one dispatch counts once
                wr.writerow({"Dispatch_Id": i + 1, "Correlation_Id": i + 1, "Grid_Size": grid,
                             "Kernel_Name": name, "Workgroup_Size": wg, "Counter_Name": counter,
                             "Counter_Value": v})


@pytest.fixture()
def segs(tmp_path):
    p = tmp_path / "segments.json"
    p.write_text(json.dumps({"segments": [{"name": "row/a", "calls": 2},
                                          {"name": "row/b", "calls": 3}],
                             "kernel_source_hash": bench.kernel_source_hash()}))
    return str(p)


def _summary(dirs, segs):
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.summarize(dirs, segs)
    return buf.getvalue()


def test_trace_summary_segments(tmp_path, segs):
    d = str(tmp_path / "trace")
    _write_trace(d)
    txt = _summary([d], segs)
    p = tmp_path / "s.md"
    p.write_text(txt)
    vals = bench.read_summary(str(p))
    # segment a: per call one 4 us and one 5 us kernel; b: one 3 us kernel
    assert vals[("trace_us", "row/a per_call")] == pytest.approx(9.0)
    assert vals[("trace_us", "row/b per_call")] == pytest.approx(3.0)
    assert vals[("trace_us", "row/a count_layout_kernel<true, 2, -1>@262144")] == \
        pytest.approx(4.0)
    # launches outside a pair of markers belong to no segment
    assert "warm" not in txt and "setup" not in txt and "after" not in txt
    assert bench._short("void moe::(anonymous namespace)::combine_kernel<8, true>(moe::Lane<2>::T "
                        "const*, float __vector(4)*, int)") == "combine_kernel<8, true>"


def test_pmc_summary_and_scaling(tmp_path, segs):
    da, db = str(tmp_path / "f"), str(tmp_path / "w")
    _write_pmc(da, "FETCH_SIZE", {"count_layout_kernel": 100.0, "combine_kernel": 50.0})
    _write_pmc(db, "WRITE_SIZE", {"count_layout_kernel": 400.0, "combine_kernel": 25.0})
    txt = _summary([da, db], segs)
    p = tmp_path / "s.md"
    p.write_text(txt)
    vals = bench.read_summary(str(p))
    assert vals[("fetch_kib", "row/a per_call")] == pytest.approx(150.0)
    assert vals[("write_kib", "row/a per_call")] == pytest.approx(425.0)
    assert vals[("fetch_kib", "row/b per_call")] == pytest.approx(50.0)
    # calibration: a 256 MiB copy whose counters read half of what it fetched
    vals[("fetch_kib", "floors/copy_256MiB per_call")] = 128 * 1024.0
    vals[("write_kib", "floors/copy_256MiB per_call")] = 256 * 1024.0
    t = bench.pmc_traffic(vals)
    assert t["factors"] == (0.5, 1.0)
    assert t[("traffic", "row/a")] == pytest.approx((150.0 / 0.5 + 425.0) * 1024)


def test_marker_count_mismatch(tmp_path, segs):
    d = str(tmp_path / "trace")
    _write_trace(d)
    data = json.load(open(segs))
    data["segments"].append({"name": "row/c", "calls": 1})
    json.dump(data, open(segs, "w"))
    with pytest.raises(SystemExit):
        _summary([d], segs)


def test_summary_rejected_for_other_sources(tmp_path):
    p = tmp_path / "s.md"
    p.write_text("kernel_source_hash: 0000000000000000\ntrace_us row/a per_call: 1.0\n")
    assert bench.read_summary(str(p)) == {}


def test_algo_bytes_standard():
    ab = bench.algo_bytes(128, 7168, 8, 256, 8, 1024)
    assert ab["dispatch"] == 1024 * (2 * 7168 + 4) + 128 * 2 * 7168
    assert ab["combine"] == 1024 * (2 * 7168 + 8) + 128 * 2 * 7168
    assert ab["total"] == 33061924


def test_multi_gpu_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stdout


@pytest.mark.parametrize("args", [["--steps", "0"], ["--warmup", "-1"]])
def test_bad_step_counts_refused(args):
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "--steps" in r.stdout


@pytest.mark.parametrize("name", ["c1", "c2", "c4"])
def test_rotating_sets_cover_twice_the_infinity_cache(name):
    """The standard-kind rows rotate over enough buffer sets that a step's
    inputs were last touched >= 512 MiB of traffic ago (twice the 256 MB
    memory-side cache), capped at 64 sets for the tiny batch."""
    import moe_inputs as mi
    from combine_moe_layout_03_amd import capi
    w = mi.by_name(name)
    nws = capi.moe_layout_workspace_bytes(capi.make_shape(w.T, w.H, w.E, w.R, w.K, w.A))
    per_set = bench.workset_bytes(w, nws)
    S = bench.n_sets(per_set)
    assert S * per_set >= 512 * 2**20 or S == 64
    # the set's own device bytes: x, routing, weights, layout arrays, receive
    # buffer, output (and workspace), each rounded to 256
    rows = w.T * w.K + w.E * (w.A - 1)
    assert per_set >= w.T * w.H * 2 * 2 + rows * w.H * 2 + w.T * w.K * 16


def test_phase_instrumentation_applies(tmp_path):
    """bench_phases.py's instrumented copy still finds every anchor in the
    current kernel sources (it stops with SystemExit otherwise), and leaves
    the library's own sources untouched."""
    import bench_phases
    before = open(os.path.join(ROOT, "combine_moe_layout_03_amd", "csrc", "fused.hip")).read()
    bench_phases.instrument(str(tmp_path))
    got = open(tmp_path / "combine_moe_layout_03_amd" / "csrc" / "fused.hip").read()
    assert got.count("STAMP(") == 11 and "moe_debug_stamps" in got and "STAMP(8)" in got
    assert "moe_debug_fstamps" in open(tmp_path / "combine_moe_layout_03_amd" / "csrc" /
                                       "floors.hip").read()
    assert open(os.path.join(ROOT, "combine_moe_layout_03_amd", "csrc", "fused.hip")).read() == before
