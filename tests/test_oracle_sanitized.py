"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only), and its OpenMP build against the normal one.

The sanitized build runs the same small pins as the normal build, in a child
process started with the ASan runtime preloaded (the Python interpreter is not
instrumented); any out-of-bounds access, use after free or undefined
behaviour aborts the child."""
import os
import subprocess
import sys

import numpy as np
import pytest

import moe_inputs as mi
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
orc = oracle.Oracle({path!r})
for chk in pins.ALL_SMALL_CHECKS:
    chk(orc)
import moe_inputs as mi
w = mi.config_c1()
pins.check_layout_invariants(orc, w, 16)
print("SANITIZED_PINS_OK", flush=True)
"""


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = out.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime for gcc here")
    path = os.path.join(str(tmp_path), "liboracle_asan.so")
    oracle.build(path, extra=("-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                              "-fno-sanitize-recover=all", "-g"))
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), path=path)
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0 and "SANITIZED_PINS_OK" in res.stdout, tail
    assert "runtime error" not in res.stderr, tail


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("name", ["c2", "bad_slots"])
def test_openmp_build_matches_serial(name):
    """The all-cores build gives the serial build's results bit for bit."""
    ser, par = oracle.get(), oracle.get_parallel()
    assert par.threads(8) == 8 and ser.threads() == 1
    if name == "c2":
        w = mi.config_c2()
    else:
        w = mi.random_case(77, 300, 136, 32, 8, 6, 1, neg_frac=0.1, dup_frac=0.1)
    lay = ser.layout(w.topk_idx, w.E, w.R, 1)
    slot = lay["slot"].copy()
    rows = lay["rows"]
    if name == "bad_slots":  # out-of-range slots set the status in every thread
        slot.reshape(-1)[::37] = rows + 5
    r1, s1 = ser.dispatch(w.x, slot, rows, fill=0x7E57)  # rows no pair writes keep the fill
    r2, s2 = par.dispatch(w.x, slot, rows, fill=0x7E57)
    assert np.array_equal(r1, r2) and s1 == s2
    if name == "bad_slots":
        assert s1 & oracle.ST_BAD_SLOT
    for mode in ("f32", "f64"):
        a = ser.combine(r1, slot, w.topk_weights, mode)
        b = par.combine(r1, slot, w.topk_weights, mode)
        assert a.keys() == b.keys()
        for k in a:
            if isinstance(a[k], np.ndarray):
                assert np.array_equal(_bits(a[k]), _bits(b[k])), (mode, k)
            else:
                assert a[k] == b[k], (mode, k)
