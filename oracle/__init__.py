"""The oracle: plain CPU definition of MoE token dispatch and combine.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may use it; the GPU product path never does.
It shares no code with the HIP library: its arithmetic lives in ``oracle.c``
(plain single-threaded C, built with ``gcc -O2 -ffp-contract=off``), and this
module only marshals numpy arrays in and out.

See ``oracle.c`` for the definitions followed and the page sections they come
from. Every function here is pinned by the ``-m "not gpu"`` tests against brute
force, library routines, closed forms and a hand-worked example.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

ST_BAD_EXPERT = 1
ST_LL_OVERFLOW = 2
ST_BAD_SLOT = 4
ST_BAD_REPLICA = 8

FP8_ROUND_SCALE = 1
FP8_UE8M0 = 2
FP8_SCALE_ROWS = 4
FP8_GROUP = 128


LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")


def build(out: str = LIB, mutant: Optional[int] = None, openmp: bool = False,
          extra: tuple = ()) -> str:
    """Compile oracle.c into a shared library (optionally with a planted
    mutant). openmp=True gives the build whose dispatch and combine token loops
    run on several threads (the CPU baseline's all-cores leg); its results are
    the same bit for bit. extra: more compiler flags (the sanitizer test)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Werror", *extra, "-o", out + ".tmp", SRC, "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    if mutant is not None:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_all() -> None:
    """The normal build and the OpenMP build."""
    build(LIB)
    build(LIB_OMP, openmp=True)


_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class Oracle:
    """ctypes view of one build of oracle.c (the normal build or a mutant)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built; run __graft_entry__.build()")
        self.path = path
        lib = C.CDLL(path)
        self.lib = lib
        lib.oracle_mutant.restype = C.c_int
        lib.oracle_threads.argtypes = [C.c_int]
        lib.oracle_threads.restype = C.c_int
        lib.oracle_bf16_from_f32.argtypes = [_P, _P, _I64]
        lib.oracle_layout.argtypes = [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                      _I64, _P]
        lib.oracle_ll_layout.argtypes = [_I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                         _P, _P]
        lib.oracle_expert_load.argtypes = [_I64, _I32, _I32, _P, _P, _P]
        lib.oracle_dispatch.argtypes = [_I64, _I32, _I32, _P, _P, _P, _I64, _P]
        lib.oracle_combine_f64.argtypes = [_I64, _I32, _I32, _P, _I64, _P, _P, _P, _P]
        lib.oracle_combine_f32.argtypes = [_I64, _I32, _I32, _P, _I64, _P, _P, _P, _P, _P]
        lib.oracle_plan_replicas.argtypes = [_I32, _I32, _I32, _P, _P, _P, _P]
        lib.oracle_reroute.argtypes = [_I64, _I32, _I32, _P, _P, _P, _I32, _P, _P]
        lib.oracle_e4m3_value.argtypes = [C.c_uint8]
        lib.oracle_e4m3_value.restype = C.c_double
        lib.oracle_e4m3_from_f32.argtypes = [_P, _P, _I64]
        lib.oracle_quantize_fp8.argtypes = [_I64, _I32, _P, _I32, _P, _P, _P]
        lib.oracle_ll_dispatch_fp8.argtypes = [_I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P,
                                               _P, _P, _P, _P, _P, _P]
        lib.oracle_quantize_fp8.restype = C.c_int
        lib.oracle_combine_masked_f32.argtypes = [_I64, _I32, _I32, _P, _I64, _P, _P, _I32, _I32,
                                                  _P, _P, _P, _P, _P]
        lib.oracle_combine_masked_f32.restype = C.c_int
        lib.oracle_accumulate_recv_stats.argtypes = [_I32, _P, _P]
        lib.oracle_rank_layout.argtypes = [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P]
        lib.oracle_rank_layout.restype = C.c_int
        lib.oracle_combine_rank_weights.argtypes = [_I64, _I32, _I32, _P, _P, _I64, _P, _P]
        lib.oracle_replica_weight_sync.argtypes = [_I32, _I64, _P, _P, _I32, _P]
        lib.oracle_replica_grad_reduce.argtypes = [_I32, _I64, _P, _P, _I32, _P]
        lib.oracle_ll_dispatch_fp8.restype = C.c_int
        for f in ("oracle_layout", "oracle_ll_layout", "oracle_expert_load", "oracle_dispatch",
                  "oracle_combine_f64", "oracle_combine_f32", "oracle_plan_replicas",
                  "oracle_reroute"):
            getattr(lib, f).restype = C.c_int

    @property
    def mutant(self) -> int:
        return int(self.lib.oracle_mutant())

    def threads(self, n: int = 0) -> int:
        """Threads of the token loops: sets them when n > 0 (OpenMP build
        only) and returns the count in force."""
        return int(self.lib.oracle_threads(int(n)))

    # -- conversions --------------------------------------------------------
    def bf16_rne(self, f: np.ndarray) -> np.ndarray:
        f = np.ascontiguousarray(f, dtype=np.float32)
        out = np.empty(f.shape, np.uint16)
        self.lib.oracle_bf16_from_f32(_ptr(f), _ptr(out), f.size)
        return out

    # -- layout -------------------------------------------------------------
    def layout(self, idx: np.ndarray, E: int, R: int, A: int = 1) -> dict:
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        T, K = idx.shape
        count = np.empty(E, np.int32)
        offset = np.empty(E + 1, np.int32)
        rtc = np.empty(R, np.int32)
        in_rank = np.empty((T, R), np.uint8)
        slot = np.empty((T, K), np.int32)
        worst = T * K + E * (A - 1)
        row_src = np.empty(max(worst, 1), np.int32)
        status = np.zeros(1, np.int32)
        rc = self.lib.oracle_layout(T, K, E, R, A, _ptr(idx), _ptr(count), _ptr(offset),
                                    _ptr(rtc), _ptr(in_rank), _ptr(slot), _ptr(row_src),
                                    row_src.size, _ptr(status))
        if rc != 0:
            raise ValueError(f"oracle_layout rejected its arguments ({rc})")
        rows = int(offset[E])
        return dict(count=count, offset=offset, rank_token_count=rtc, is_token_in_rank=in_rank,
                    slot=slot, row_src=row_src[:rows].copy(), rows=rows,
                    status=int(status[0]))

    def ll_layout(self, idx: np.ndarray, E: int, R: int, M: int, src_rank: int = 0) -> dict:
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        T, K = idx.shape
        recv_count = np.empty(E, np.int32)
        rtc = np.empty(R, np.int32)
        in_rank = np.empty((T, R), np.uint8)
        slot = np.empty((T, K), np.int32)
        row_src = np.empty(E * M, np.int32)
        status = np.zeros(1, np.int32)
        rc = self.lib.oracle_ll_layout(T, K, E, R, M, src_rank, _ptr(idx), _ptr(recv_count),
                                       _ptr(rtc), _ptr(in_rank), _ptr(slot), _ptr(row_src),
                                       _ptr(status))
        if rc != 0:
            raise ValueError(f"oracle_ll_layout rejected its arguments ({rc})")
        return dict(recv_count=recv_count, rank_token_count=rtc, is_token_in_rank=in_rank,
                    slot=slot, row_src=row_src, rows=E * R * M, status=int(status[0]))

    def expert_load(self, idx: np.ndarray, E: int) -> tuple:
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        T, K = idx.shape
        load = np.empty(E, np.int32)
        status = np.zeros(1, np.int32)
        rc = self.lib.oracle_expert_load(T, K, E, _ptr(idx), _ptr(load), _ptr(status))
        if rc != 0:
            raise ValueError(rc)
        return load, int(status[0])

    # -- dispatch / combine -------------------------------------------------
    def dispatch(self, x: np.ndarray, slot: np.ndarray, rows: int,
                 fill: Optional[int] = None, out: Optional[np.ndarray] = None) -> tuple:
        x = np.ascontiguousarray(x, dtype=np.uint16)
        slot = np.ascontiguousarray(slot, dtype=np.int32)
        T, H = x.shape
        K = slot.shape[1]
        if out is None:
            out = np.empty((rows, H), np.uint16) if fill is None else \
                np.full((rows, H), fill, np.uint16)
        status = np.zeros(1, np.int32)
        self.lib.oracle_dispatch(T, H, K, _ptr(x), _ptr(slot), _ptr(out), rows, _ptr(status))
        return out, int(status[0])

    def combine(self, y: np.ndarray, slot: np.ndarray, w: Optional[np.ndarray],
                acc: str = "f64") -> dict:
        y = np.ascontiguousarray(y, dtype=np.uint16)
        slot = np.ascontiguousarray(slot, dtype=np.int32)
        T, K = slot.shape
        rows, H = y.shape
        if w is not None:
            w = np.ascontiguousarray(w, dtype=np.float32)
            assert w.shape == (T, K)
        status = np.zeros(1, np.int32)
        if acc == "f64":
            out = np.empty((T, H), np.float64)
            self.lib.oracle_combine_f64(T, H, K, _ptr(y), rows, _ptr(slot), _ptr(w), _ptr(out),
                                        _ptr(status))
            return dict(out_f64=out, status=int(status[0]))
        if acc == "f32":
            o32 = np.empty((T, H), np.float32)
            o16 = np.empty((T, H), np.uint16)
            self.lib.oracle_combine_f32(T, H, K, _ptr(y), rows, _ptr(slot), _ptr(w), _ptr(o32),
                                        _ptr(o16), _ptr(status))
            return dict(out_f32=o32, out_bf16=o16, status=int(status[0]))
        raise ValueError(acc)

    # -- FP8 ----------------------------------------------------------------
    def e4m3_value(self, codes: np.ndarray) -> np.ndarray:
        """Values (float64) of E4M3 codes; NaN for the two NaN codes."""
        codes = np.asarray(codes, dtype=np.uint8)
        return np.array([self.lib.oracle_e4m3_value(int(c)) for c in codes.ravel()],
                        np.float64).reshape(codes.shape)

    def e4m3_from_f32(self, v: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float32)
        out = np.empty(v.shape, np.uint8)
        self.lib.oracle_e4m3_from_f32(_ptr(v), _ptr(out), v.size)
        return out

    def quantize_fp8(self, x: np.ndarray, flags: int = 0) -> dict:
        """Per-token E4M3 cast with one scale per 128 channels (see oracle.c)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        T, H = x.shape
        G = H // FP8_GROUP
        q = np.empty((T, H), np.uint8)
        scale = np.empty((T, G), np.float32)
        ue = np.empty((T, max(G // 4, 1)), np.int32) if flags & FP8_UE8M0 else None
        rc = self.lib.oracle_quantize_fp8(T, H, _ptr(x), flags, _ptr(q), _ptr(scale), _ptr(ue))
        if rc != 0:
            raise ValueError(f"oracle_quantize_fp8 rejected its arguments ({rc})")
        return dict(q=q, scale=scale, ue8m0=ue)

    def ll_dispatch_fp8(self, qz: dict, slot: np.ndarray, E: int, R: int, M: int, flags: int = 0,
                        fill_q: int = 0, fill_scale: float = 0.0, fill_ue: int = 0) -> dict:
        """Scatter quantized rows and their scales (column-major [E, G, R*M], or
        row-major [rows, G] with FP8_SCALE_ROWS) to the low-latency padded
        layout; untouched entries keep the fill values."""
        q, scale, ue = qz["q"], qz["scale"], qz["ue8m0"]
        slot = np.ascontiguousarray(slot, dtype=np.int32)
        T, H = q.shape
        K = slot.shape[1]
        G = H // FP8_GROUP
        rows = E * R * M
        recv_q = np.full((rows, H), fill_q, np.uint8)
        if flags & FP8_SCALE_ROWS:  # row-major option: [rows, G] / [rows, G/4]
            recv_s = np.full((rows, G), fill_scale, np.float32)
            recv_u = np.full((rows, max(G // 4, 1)), fill_ue, np.int32) \
                if flags & FP8_UE8M0 else None
        else:  # the page's column-major last two dimensions
            recv_s = np.full((E, G, R * M), fill_scale, np.float32)
            recv_u = np.full((E, max(G // 4, 1), R * M), fill_ue, np.int32) \
                if flags & FP8_UE8M0 else None
        status = np.zeros(1, np.int32)
        rc = self.lib.oracle_ll_dispatch_fp8(T, H, K, E, R, M, flags, _ptr(slot), _ptr(q),
                                             _ptr(scale), _ptr(ue), _ptr(recv_q), _ptr(recv_s),
                                             _ptr(recv_u), _ptr(status))
        if rc != 0:
            raise ValueError(f"oracle_ll_dispatch_fp8 rejected its arguments ({rc})")
        return dict(recv_q=recv_q, recv_scale=recv_s, recv_ue8m0=recv_u, status=int(status[0]))

    def dispatch_fp8_tuple(self, q: np.ndarray, scale: np.ndarray, slot: np.ndarray, rows: int,
                           fill16: int = 0) -> tuple:
        """Buffer.dispatch with x = (E4M3 rows, float scales): both members of
        the tuple are copied row by row to the pair's slot -- the plain row
        copy, applied to the code bytes and to the scale words (viewed as
        16-bit units). Untouched rows hold the 16-bit pattern fill16."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        T, H = q.shape
        G = scale.shape[1]
        rq, st1 = self.dispatch(q.view(np.uint16), slot, rows, fill=fill16)
        rs, st2 = self.dispatch(scale.view(np.uint16), slot, rows, fill=fill16)
        return rq.view(np.uint8).reshape(rows, H), rs.view(np.float32).reshape(rows, G), st1 | st2

    def combine_masked(self, y: np.ndarray, slot: np.ndarray, idx: np.ndarray, E: int, R: int,
                       mask: np.ndarray, w: Optional[np.ndarray]) -> dict:
        """Combine (float, ascending k) skipping pairs whose expert's rank is masked."""
        y = np.ascontiguousarray(y, dtype=np.uint16)
        slot = np.ascontiguousarray(slot, dtype=np.int32)
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        mask = np.ascontiguousarray(mask, dtype=np.int32)
        T, K = slot.shape
        rows, H = y.shape
        if w is not None:
            w = np.ascontiguousarray(w, dtype=np.float32)
        o32 = np.empty((T, H), np.float32)
        o16 = np.empty((T, H), np.uint16)
        status = np.zeros(1, np.int32)
        rc = self.lib.oracle_combine_masked_f32(T, H, K, _ptr(y), rows, _ptr(slot), _ptr(idx), E,
                                                R, _ptr(mask), _ptr(w), _ptr(o32), _ptr(o16),
                                                _ptr(status))
        if rc != 0:
            raise ValueError(rc)
        return dict(out_f32=o32, out_bf16=o16, status=int(status[0]))

    def accumulate_recv_stats(self, recv_count: np.ndarray, stats: np.ndarray) -> np.ndarray:
        """stats += recv_count (cumulative_local_expert_recv_stats); returns stats."""
        rc_ = np.ascontiguousarray(recv_count, dtype=np.int32)
        st = np.ascontiguousarray(stats, dtype=np.int32).copy()
        self.lib.oracle_accumulate_recv_stats(rc_.size, _ptr(rc_), _ptr(st))
        return st

    # -- normal mode: one row per (token, rank) ----------------------------
    def rank_layout(self, idx: np.ndarray, E: int, R: int, A: int = 1,
                    w: Optional[np.ndarray] = None) -> dict:
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        T, K = idx.shape
        worst = max(T * min(K, R), 1)
        rank_slot = np.empty((T, R), np.int32)
        rank_offset = np.empty(R + 1, np.int32)
        recv_src = np.empty(worst, np.int32)
        recv_idx = np.empty((worst, K), np.int64)
        recv_w = np.empty((worst, K), np.float32)
        rec = np.empty(E, np.int32)
        status = np.zeros(1, np.int32)
        if w is not None:
            w = np.ascontiguousarray(w, dtype=np.float32)
        rc = self.lib.oracle_rank_layout(T, K, E, R, A, _ptr(idx), _ptr(w), _ptr(rank_slot),
                                         _ptr(rank_offset), _ptr(recv_src), _ptr(recv_idx),
                                         _ptr(recv_w), _ptr(rec), _ptr(status))
        if rc != 0:
            raise ValueError(f"oracle_rank_layout rejected its arguments ({rc})")
        rows = int(rank_offset[R])
        return dict(rank_slot=rank_slot, rank_offset=rank_offset, recv_src=recv_src[:rows].copy(),
                    recv_topk_idx=recv_idx[:rows].copy(),
                    recv_topk_weights=recv_w[:rows].copy() if w is not None else None,
                    recv_expert_count=rec, rows=rows, status=int(status[0]))

    def combine_rank_weights(self, rank_slot: np.ndarray, recv_w: np.ndarray) -> tuple:
        rank_slot = np.ascontiguousarray(rank_slot, dtype=np.int32)
        recv_w = np.ascontiguousarray(recv_w, dtype=np.float32)
        T, R = rank_slot.shape
        rows, K = recv_w.shape
        out = np.empty((T, K), np.float32)
        status = np.zeros(1, np.int32)
        self.lib.oracle_combine_rank_weights(T, K, R, _ptr(rank_slot), _ptr(recv_w), rows,
                                             _ptr(out), _ptr(status))
        return out, int(status[0])

    # -- replicas -----------------------------------------------------------
    def plan_replicas(self, load: np.ndarray, R: int, C_: int) -> dict:
        load = np.ascontiguousarray(load, dtype=np.int32)
        E = load.size
        rc_ = np.empty(E, np.int32)
        rp = np.empty((E, 2), np.int32)
        p2l = np.empty(E + C_, np.int32)
        rc = self.lib.oracle_plan_replicas(E, R, C_, _ptr(load), _ptr(rc_), _ptr(rp), _ptr(p2l))
        if rc != 0:
            raise ValueError(f"oracle_plan_replicas rejected its arguments ({rc})")
        return dict(replica_count=rc_, replica_phys=rp, phys_to_logical=p2l, E_phys=E + C_,
                    L_phys=E // R + C_ // R)

    def replica_weight_sync(self, w: np.ndarray, replica_count: np.ndarray,
                            replica_phys: np.ndarray) -> np.ndarray:
        """Copy of w [E_phys, S] (bf16 bits) after the replica weight sync."""
        w = np.ascontiguousarray(w, dtype=np.uint16).copy()
        rc = np.ascontiguousarray(replica_count, np.int32)
        rp = np.ascontiguousarray(replica_phys, np.int32)
        res = self.lib.oracle_replica_weight_sync(rc.size, w.shape[1], _ptr(rc), _ptr(rp),
                                                  w.shape[0], _ptr(w))
        if res != 0:
            raise ValueError(res)
        return w

    def replica_grad_reduce(self, g: np.ndarray, replica_count: np.ndarray,
                            replica_phys: np.ndarray) -> np.ndarray:
        """Copy of g [E_phys, S] (f32) after the replica gradient reduction."""
        g = np.ascontiguousarray(g, dtype=np.float32).copy()
        rc = np.ascontiguousarray(replica_count, np.int32)
        rp = np.ascontiguousarray(replica_phys, np.int32)
        res = self.lib.oracle_replica_grad_reduce(rc.size, g.shape[1], _ptr(rc), _ptr(rp),
                                                  g.shape[0], _ptr(g))
        if res != 0:
            raise ValueError(res)
        return g

    def reroute(self, idx: np.ndarray, E: int, replica_count: np.ndarray,
                replica_phys: np.ndarray, E_phys: int) -> tuple:
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        T, K = idx.shape
        out = np.empty((T, K), np.int64)
        status = np.zeros(1, np.int32)
        rc = self.lib.oracle_reroute(T, K, E, _ptr(idx),
                                     _ptr(np.ascontiguousarray(replica_count, np.int32)),
                                     _ptr(np.ascontiguousarray(replica_phys, np.int32)),
                                     E_phys, _ptr(out), _ptr(status))
        if rc != 0:
            raise ValueError(rc)
        return out, int(status[0])


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The normal (unmutated) oracle build; built on first use if absent."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = Oracle(LIB)
    return _default


_parallel: Optional[Oracle] = None


def get_parallel() -> Oracle:
    """The OpenMP build (same results; dispatch and combine split over
    tokens); built on first use if absent."""
    global _parallel
    if _parallel is None:
        if not os.path.exists(LIB_OMP):
            build(LIB_OMP, openmp=True)
        _parallel = Oracle(LIB_OMP)
    return _parallel
