"""ctypes binding of libmoe_ep.so: one Python function per C entry point, same
names, argument marshalling only (torch tensors -> device pointers, the current
torch stream -> hipStream_t). Every step runs in the library's HIP kernels;
there is no fallback: if the library is not built, importing this module
raises.

The checks here are the ones the C ABI cannot make itself: that each tensor is
on the GPU, contiguous, of the right dtype and large enough for what the call
will write or read.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ep.so")

MOE_ABI_VERSION = 5  # the version the binding is written against
MOE_STATIC_SCRATCH_BYTES = 4 << 20

MOE_STATUS_BAD_EXPERT = 1
MOE_STATUS_LL_OVERFLOW = 2
MOE_STATUS_BAD_SLOT = 4
MOE_STATUS_BAD_REPLICA = 8

MOE_FP8_ROUND_SCALE = 1
MOE_FP8_UE8M0 = 2
MOE_FP8_SCALE_ROWS = 4
FP8_GROUP = 128


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {moe_strerror(code)} ({code})")
        self.code = code


class moe_shape(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("E", C.c_int32), ("R", C.c_int32),
                ("K", C.c_int32), ("A", C.c_int32)]

    def __repr__(self):
        return (f"moe_shape(T={self.T}, H={self.H}, E={self.E}, R={self.R}, K={self.K}, "
                f"A={self.A})")


class moe_layout_t(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("count", "offset", "rank_token_count",
                                          "is_token_in_rank", "slot", "row_src", "status",
                                          "recv_stats")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m combine_moe_layout_03_amd.build`"
                          " (or __graft_entry__.build())")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "moe_abi_version": (C.c_int, []),
        "moe_strerror": (C.c_char_p, [C.c_int]),
        "moe_recv_rows_worst": (I64, [P]),
        "moe_ll_recv_rows": (I64, [I32, I32, I32]),
        "moe_layout_workspace_bytes": (SZ, [P]),
        "moe_layout": (C.c_int, [P, P, P, P, SZ, P]),
        "moe_ll_layout": (C.c_int, [P, I32, I32, P, P, P, SZ, P]),
        "moe_layout_dispatch": (C.c_int, [P, P, P, P, P, I64, P, SZ, P]),
        "moe_layout_dispatch_static": (C.c_int, [P, P, P, P, P, I64, P]),
        "moe_ll_layout_dispatch": (C.c_int, [P, I32, I32, P, P, P, P, I64, P, SZ, P]),
        "moe_expert_load": (C.c_int, [I32, I32, I32, P, P, P, P]),
        "moe_dispatch": (C.c_int, [P, P, P, P, I64, P, P]),
        "moe_combine": (C.c_int, [P, P, I64, P, P, P, P, P, P]),
        "moe_plan_replicas": (C.c_int, [I32, I32, I32, P, P, P, P, P]),
        "moe_reroute": (C.c_int, [I32, I32, I32, P, P, P, I32, P, P, P]),
        "moe_quantize_fp8": (C.c_int, [I32, I32, P, P, P, I32, P]),
        "moe_ll_layout_dispatch_fp8": (C.c_int, [P, I32, I32, P, P, P, P, P, I64, I32, P, SZ,
                                                 P]),
        "moe_ll_dispatch_fp8": (C.c_int, [P, I32, P, P, P, P, I64, I32, P, P]),
        "moe_dispatch_fp8": (C.c_int, [P, P, P, P, P, P, I64, P, P]),
        "moe_combine_masked": (C.c_int, [P, P, I64, P, P, P, P, P, P, P, P]),
        "moe_rank_recv_rows_worst": (I64, [P]),
        "moe_rank_layout": (C.c_int, [P, P, P, P, I64, P]),
        "moe_rank_dispatch": (C.c_int, [P, P, P, P, I64, P, P]),
        "moe_rank_layout_dispatch": (C.c_int, [P, P, P, P, I64, P, P, I64, P]),
        "moe_rank_combine": (C.c_int, [P, P, I64, P, P, P, P, P, P, P]),
        "moe_replica_weight_sync": (C.c_int, [I32, I32, I64, P, P, P, P, P]),
        "moe_replica_grad_reduce": (C.c_int, [I32, I32, I64, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("moe_abi_version", "moe_strerror", "moe_recv_rows_worst", "moe_ll_recv_rows",
            "moe_layout_workspace_bytes", "moe_layout", "moe_ll_layout", "moe_layout_dispatch",
            "moe_layout_dispatch_static",
            "moe_ll_layout_dispatch", "moe_expert_load",
            "moe_dispatch", "moe_combine", "moe_plan_replicas", "moe_reroute",
            "moe_quantize_fp8", "moe_ll_layout_dispatch_fp8", "moe_ll_dispatch_fp8",
            "moe_dispatch_fp8", "moe_combine_masked", "moe_rank_recv_rows_worst",
            "moe_rank_layout", "moe_rank_dispatch", "moe_rank_layout_dispatch",
            "moe_rank_combine",
            "moe_replica_weight_sync", "moe_replica_grad_reduce")


def lib():
    return _lib


# -- marshalling helpers -----------------------------------------------------

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)
_FP8_CODES = (torch.uint8, torch.int8, torch.float8_e4m3fn)


def fp8_scale_cols(H: int, flags: int) -> int:
    """Scale entries per row: one float per 128 channels, or one UE8M0 word per 512."""
    return H // (4 * FP8_GROUP) if flags & MOE_FP8_UE8M0 else H // FP8_GROUP


def _ll_scale_numel(E: int, R: int, M: int, H: int, recv_rows: int, flags: int) -> int:
    """Scale entries the low-latency FP8 calls may write: [E][cols][R*M]
    column-major, or [recv_rows][cols] with MOE_FP8_SCALE_ROWS."""
    if not recv_rows:
        return 0
    cols = fp8_scale_cols(H, flags)
    return int(recv_rows) * cols if flags & MOE_FP8_SCALE_ROWS else E * cols * R * int(M)


def _fp8_scale_dtypes(flags: int):
    return (torch.int32,) if flags & MOE_FP8_UE8M0 else (torch.float32,)


def _dev(t: Optional[torch.Tensor], name: str, dtypes, min_numel: int = 0, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    return C.c_void_p(t.data_ptr()) if t.numel() > 0 else None


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise MoeError(fn, rc)
    return rc


def make_shape(T: int, H: int, E: int, R: int, K: int, A: int = 1) -> moe_shape:
    return moe_shape(int(T), int(H), int(E), int(R), int(K), int(A))


@dataclass
class LayoutBuffers:
    """Device arrays of a layout (the dispatch "handle"). Optional ones may be None."""

    count: torch.Tensor
    offset: Optional[torch.Tensor]
    slot: torch.Tensor
    rank_token_count: Optional[torch.Tensor] = None
    is_token_in_rank: Optional[torch.Tensor] = None
    row_src: Optional[torch.Tensor] = None
    status: Optional[torch.Tensor] = None
    recv_stats: Optional[torch.Tensor] = None  # [E] int32, cumulative (+= count)

    @staticmethod
    def empty(shape: moe_shape, device, ll_M: Optional[int] = None, extras: bool = True,
              status: bool = True, rank_tables: bool = True) -> "LayoutBuffers":
        """extras: the optional outputs; rank_tables=False leaves out the
        per-rank token counts and the token-rank table among them (what the
        low-latency dispatch does not return)."""
        T, E, R, K = shape.T, shape.E, shape.R, shape.K
        i32 = dict(dtype=torch.int32, device=device)
        if ll_M is None:
            rows_src = max(int(moe_recv_rows_worst(shape)), 1)
        else:
            rows_src = E * ll_M
        return LayoutBuffers(
            count=torch.empty(E, **i32),
            offset=torch.empty(E + 1, **i32),
            slot=torch.empty(T * K, **i32),
            rank_token_count=torch.empty(R, **i32) if extras and rank_tables else None,
            is_token_in_rank=torch.empty(T * R, dtype=torch.uint8, device=device)
            if extras and rank_tables else None,
            row_src=torch.empty(rows_src, **i32) if extras else None,
            status=torch.zeros(1, **i32) if status else None,
        )

    def _struct(self, shape: moe_shape, ll_M: Optional[int]) -> moe_layout_t:
        T, E, R, K = shape.T, shape.E, shape.R, shape.K
        i32 = (torch.int32,)
        rs_need = E * ll_M if ll_M is not None else max(int(moe_recv_rows_worst(shape)), 0)
        return moe_layout_t(
            _dev(self.count, "count", i32, E),
            _dev(self.offset, "offset", i32, E + 1, optional=ll_M is not None),
            _dev(self.rank_token_count, "rank_token_count", i32, R, optional=True),
            _dev(self.is_token_in_rank, "is_token_in_rank", (torch.uint8, torch.bool), T * R,
                 optional=True),
            _dev(self.slot, "slot", i32, T * K),
            _dev(self.row_src, "row_src", i32, rs_need, optional=True),
            _dev(self.status, "status", i32, 1, optional=True),
            _dev(self.recv_stats, "recv_stats", i32, E, optional=True),
        )


class moe_rank_layout_t(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("rank_slot", "rank_offset", "recv_src",
                                          "recv_topk_idx", "recv_topk_weights",
                                          "recv_expert_count", "status")]


@dataclass
class RankLayoutBuffers:
    """Device arrays of a normal-mode layout (one row per (token, rank))."""

    rank_slot: torch.Tensor
    rank_offset: torch.Tensor
    recv_src: Optional[torch.Tensor] = None
    recv_topk_idx: Optional[torch.Tensor] = None
    recv_topk_weights: Optional[torch.Tensor] = None
    recv_expert_count: Optional[torch.Tensor] = None
    status: Optional[torch.Tensor] = None
    cap: int = 0

    @staticmethod
    def empty(shape: "moe_shape", device, weights: bool = True, cap: Optional[int] = None):
        T, E, R, K = shape.T, shape.E, shape.R, shape.K
        cap = int(moe_rank_recv_rows_worst(shape)) if cap is None else int(cap)
        n = max(cap, 1)
        i32 = dict(dtype=torch.int32, device=device)
        return RankLayoutBuffers(
            rank_slot=torch.empty(T * R, **i32), rank_offset=torch.empty(R + 1, **i32),
            recv_src=torch.empty(n, **i32),
            recv_topk_idx=torch.empty(n * K, dtype=torch.int64, device=device),
            recv_topk_weights=torch.empty(n * K, dtype=torch.float32, device=device)
            if weights else None,
            recv_expert_count=torch.empty(E, **i32), status=torch.zeros(1, **i32), cap=cap)

    def _struct(self, shape: "moe_shape") -> moe_rank_layout_t:
        T, E, R, K = shape.T, shape.E, shape.R, shape.K
        i32 = (torch.int32,)
        return moe_rank_layout_t(
            _dev(self.rank_slot, "rank_slot", i32, T * R),
            _dev(self.rank_offset, "rank_offset", i32, R + 1),
            _dev(self.recv_src, "recv_src", i32, self.cap, optional=True),
            _dev(self.recv_topk_idx, "recv_topk_idx", (torch.int64,), self.cap * K, optional=True),
            _dev(self.recv_topk_weights, "recv_topk_weights", (torch.float32,), self.cap * K,
                 optional=True),
            _dev(self.recv_expert_count, "recv_expert_count", i32, E, optional=True),
            _dev(self.status, "status", i32, 1, optional=True))


# -- entry points (same names as the C ABI) -----------------------------------

def moe_abi_version() -> int:
    return int(_lib.moe_abi_version())


def moe_strerror(code: int) -> str:
    return _lib.moe_strerror(int(code)).decode()


def moe_recv_rows_worst(shape: moe_shape) -> int:
    return int(_lib.moe_recv_rows_worst(C.byref(shape)))


def moe_ll_recv_rows(E: int, R: int, M: int) -> int:
    return int(_lib.moe_ll_recv_rows(E, R, M))


def moe_layout_workspace_bytes(shape: moe_shape) -> int:
    return int(_lib.moe_layout_workspace_bytes(C.byref(shape)))


def _ws(ws: Optional[torch.Tensor], shape: moe_shape):
    need = moe_layout_workspace_bytes(shape)
    if need == 0:
        return None, 0
    if ws is None:
        raise ValueError(f"this shape needs a {need}-byte device workspace")
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = ws.numel() * ws.element_size()
    return C.c_void_p(ws.data_ptr()), nbytes


def moe_layout(shape: moe_shape, topk_idx: torch.Tensor, out: LayoutBuffers,
               ws: Optional[torch.Tensor] = None, stream=None) -> int:
    idx = _dev(topk_idx, "topk_idx", (torch.int64,), shape.T * shape.K)
    st = out._struct(shape, None)
    wsp, wsn = _ws(ws, shape)
    return _check("moe_layout", _lib.moe_layout(C.byref(shape), idx, C.byref(st), wsp, wsn,
                                                _stream(stream)))


def moe_ll_layout(shape: moe_shape, M: int, src_rank: int, topk_idx: torch.Tensor,
                  out: LayoutBuffers, ws: Optional[torch.Tensor] = None, stream=None) -> int:
    idx = _dev(topk_idx, "topk_idx", (torch.int64,), shape.T * shape.K)
    st = out._struct(shape, int(M))
    wsp, wsn = _ws(ws, shape)
    return _check("moe_ll_layout", _lib.moe_ll_layout(C.byref(shape), int(M), int(src_rank), idx,
                                                      C.byref(st), wsp, wsn, _stream(stream)))


def moe_layout_dispatch(shape: moe_shape, topk_idx: torch.Tensor, out: LayoutBuffers,
                        x: torch.Tensor, recv_x: torch.Tensor, recv_rows: int,
                        ws: Optional[torch.Tensor] = None, stream=None) -> int:
    T, H, K = shape.T, shape.H, shape.K
    idx = _dev(topk_idx, "topk_idx", (torch.int64,), T * K)
    st = out._struct(shape, None)
    wsp, wsn = _ws(ws, shape)
    return _check("moe_layout_dispatch", _lib.moe_layout_dispatch(
        C.byref(shape), idx, C.byref(st), _dev(x, "x", _BF16_LIKE, T * H),
        _dev(recv_x, "recv_x", _BF16_LIKE, int(recv_rows) * H), int(recv_rows), wsp, wsn,
        _stream(stream)))


def moe_layout_dispatch_static(shape: moe_shape, topk_idx: torch.Tensor, out: LayoutBuffers,
                               x: torch.Tensor, recv_x: torch.Tensor, recv_rows: int,
                               stream=None) -> int:
    """moe_layout_dispatch without a workspace argument: the library's static
    per-GPU scratch serves the batches that need one (nothing is allocated)."""
    T, H, K = shape.T, shape.H, shape.K
    idx = _dev(topk_idx, "topk_idx", (torch.int64,), T * K)
    st = out._struct(shape, None)
    return _check("moe_layout_dispatch_static", _lib.moe_layout_dispatch_static(
        C.byref(shape), idx, C.byref(st), _dev(x, "x", _BF16_LIKE, T * H),
        _dev(recv_x, "recv_x", _BF16_LIKE, int(recv_rows) * H), int(recv_rows),
        _stream(stream)))


def moe_ll_layout_dispatch(shape: moe_shape, M: int, src_rank: int, topk_idx: torch.Tensor,
                           out: LayoutBuffers, x: torch.Tensor, recv_x: torch.Tensor,
                           recv_rows: int, ws: Optional[torch.Tensor] = None,
                           stream=None) -> int:
    T, H, K = shape.T, shape.H, shape.K
    idx = _dev(topk_idx, "topk_idx", (torch.int64,), T * K)
    st = out._struct(shape, int(M))
    wsp, wsn = _ws(ws, shape)
    return _check("moe_ll_layout_dispatch", _lib.moe_ll_layout_dispatch(
        C.byref(shape), int(M), int(src_rank), idx, C.byref(st),
        _dev(x, "x", _BF16_LIKE, T * H), _dev(recv_x, "recv_x", _BF16_LIKE, int(recv_rows) * H),
        int(recv_rows), wsp, wsn, _stream(stream)))


def moe_expert_load(T: int, K: int, E: int, topk_idx: torch.Tensor, load: torch.Tensor,
                    status: Optional[torch.Tensor] = None, stream=None) -> int:
    idx = _dev(topk_idx, "topk_idx", (torch.int64,), T * K)
    return _check("moe_expert_load", _lib.moe_expert_load(
        T, K, E, idx, _dev(load, "load", (torch.int32,), E),
        _dev(status, "status", (torch.int32,), 1, optional=True), _stream(stream)))


def moe_dispatch(shape: moe_shape, x: torch.Tensor, slot: torch.Tensor, recv_x: torch.Tensor,
                 recv_rows: int, status: Optional[torch.Tensor] = None, stream=None) -> int:
    T, H, K = shape.T, shape.H, shape.K
    return _check("moe_dispatch", _lib.moe_dispatch(
        C.byref(shape), _dev(x, "x", _BF16_LIKE, T * H), _dev(slot, "slot", (torch.int32,), T * K),
        _dev(recv_x, "recv_x", _BF16_LIKE, int(recv_rows) * H), int(recv_rows),
        _dev(status, "status", (torch.int32,), 1, optional=True), _stream(stream)))


def moe_combine(shape: moe_shape, y: torch.Tensor, recv_rows: int, slot: torch.Tensor,
                topk_weights: Optional[torch.Tensor], out: torch.Tensor,
                out_f32: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                stream=None) -> int:
    T, H, K = shape.T, shape.H, shape.K
    return _check("moe_combine", _lib.moe_combine(
        C.byref(shape), _dev(y, "y", _BF16_LIKE, int(recv_rows) * H), int(recv_rows),
        _dev(slot, "slot", (torch.int32,), T * K),
        _dev(topk_weights, "topk_weights", (torch.float32,), T * K, optional=True),
        _dev(out, "out", _BF16_LIKE, T * H),
        _dev(out_f32, "out_f32", (torch.float32,), T * H, optional=True),
        _dev(status, "status", (torch.int32,), 1, optional=True), _stream(stream)))


def moe_combine_masked(shape: moe_shape, y: torch.Tensor, recv_rows: int, slot: torch.Tensor,
                       topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                       rank_mask: torch.Tensor, out: torch.Tensor,
                       out_f32: Optional[torch.Tensor] = None,
                       status: Optional[torch.Tensor] = None, stream=None) -> int:
    T, H, K = shape.T, shape.H, shape.K
    return _check("moe_combine_masked", _lib.moe_combine_masked(
        C.byref(shape), _dev(y, "y", _BF16_LIKE, int(recv_rows) * H), int(recv_rows),
        _dev(slot, "slot", (torch.int32,), T * K),
        _dev(topk_idx, "topk_idx", (torch.int64,), T * K),
        _dev(topk_weights, "topk_weights", (torch.float32,), T * K, optional=True),
        _dev(rank_mask, "rank_mask", (torch.int32,), shape.R),
        _dev(out, "out", _BF16_LIKE, T * H),
        _dev(out_f32, "out_f32", (torch.float32,), T * H, optional=True),
        _dev(status, "status", (torch.int32,), 1, optional=True), _stream(stream)))


def moe_rank_recv_rows_worst(shape: moe_shape) -> int:
    return int(_lib.moe_rank_recv_rows_worst(C.byref(shape)))


def moe_rank_layout(shape: moe_shape, topk_idx: torch.Tensor,
                    topk_weights: Optional[torch.Tensor], out: RankLayoutBuffers,
                    stream=None) -> int:
    T, K = shape.T, shape.K
    st = out._struct(shape)
    return _check("moe_rank_layout", _lib.moe_rank_layout(
        C.byref(shape), _dev(topk_idx, "topk_idx", (torch.int64,), T * K),
        _dev(topk_weights, "topk_weights", (torch.float32,), T * K, optional=True),
        C.byref(st), int(out.cap), _stream(stream)))


def moe_rank_dispatch(shape: moe_shape, x: torch.Tensor, rank_slot: torch.Tensor,
                      recv_x: torch.Tensor, recv_rows: int, status: Optional[torch.Tensor] = None,
                      stream=None) -> int:
    T, H, R = shape.T, shape.H, shape.R
    return _check("moe_rank_dispatch", _lib.moe_rank_dispatch(
        C.byref(shape), _dev(x, "x", _BF16_LIKE, T * H),
        _dev(rank_slot, "rank_slot", (torch.int32,), T * R),
        _dev(recv_x, "recv_x", _BF16_LIKE, int(recv_rows) * H), int(recv_rows),
        _dev(status, "status", (torch.int32,), 1, optional=True), _stream(stream)))


def moe_rank_layout_dispatch(shape: moe_shape, topk_idx: torch.Tensor,
                             topk_weights: Optional[torch.Tensor], out: RankLayoutBuffers,
                             x: torch.Tensor, recv_x: torch.Tensor, recv_rows: int,
                             stream=None) -> int:
    T, K, H = shape.T, shape.K, shape.H
    st = out._struct(shape)
    return _check("moe_rank_layout_dispatch", _lib.moe_rank_layout_dispatch(
        C.byref(shape), _dev(topk_idx, "topk_idx", (torch.int64,), T * K),
        _dev(topk_weights, "topk_weights", (torch.float32,), T * K, optional=True),
        C.byref(st), int(out.cap), _dev(x, "x", _BF16_LIKE, T * H),
        _dev(recv_x, "recv_x", _BF16_LIKE, int(recv_rows) * H), int(recv_rows),
        _stream(stream)))


def moe_rank_combine(shape: moe_shape, y: torch.Tensor, recv_rows: int, rank_slot: torch.Tensor,
                     recv_topk_weights: Optional[torch.Tensor], out: torch.Tensor,
                     out_f32: Optional[torch.Tensor] = None,
                     out_topk_weights: Optional[torch.Tensor] = None,
                     status: Optional[torch.Tensor] = None, stream=None) -> int:
    T, H, R, K = shape.T, shape.H, shape.R, shape.K
    return _check("moe_rank_combine", _lib.moe_rank_combine(
        C.byref(shape), _dev(y, "y", _BF16_LIKE, int(recv_rows) * H), int(recv_rows),
        _dev(rank_slot, "rank_slot", (torch.int32,), T * R),
        _dev(recv_topk_weights, "recv_topk_weights", (torch.float32,), int(recv_rows) * K,
             optional=True),
        _dev(out, "out", _BF16_LIKE, T * H),
        _dev(out_f32, "out_f32", (torch.float32,), T * H, optional=True),
        _dev(out_topk_weights, "out_topk_weights", (torch.float32,), T * K, optional=True),
        _dev(status, "status", (torch.int32,), 1, optional=True), _stream(stream)))


def moe_plan_replicas(E: int, R: int, C_: int, load: torch.Tensor, replica_count: torch.Tensor,
                      replica_phys: torch.Tensor, phys_to_logical: torch.Tensor,
                      stream=None) -> int:
    i32 = (torch.int32,)
    return _check("moe_plan_replicas", _lib.moe_plan_replicas(
        E, R, C_, _dev(load, "load", i32, E), _dev(replica_count, "replica_count", i32, E),
        _dev(replica_phys, "replica_phys", i32, 2 * E),
        _dev(phys_to_logical, "phys_to_logical", i32, E + C_), _stream(stream)))


def moe_reroute(T: int, K: int, E: int, topk_idx: torch.Tensor, replica_count: torch.Tensor,
                replica_phys: torch.Tensor, E_phys: int, phys_idx: torch.Tensor,
                status: Optional[torch.Tensor] = None, stream=None) -> int:
    i32 = (torch.int32,)
    return _check("moe_reroute", _lib.moe_reroute(
        T, K, E, _dev(topk_idx, "topk_idx", (torch.int64,), T * K),
        _dev(replica_count, "replica_count", i32, E),
        _dev(replica_phys, "replica_phys", i32, 2 * E), int(E_phys),
        _dev(phys_idx, "phys_idx", (torch.int64,), T * K),
        _dev(status, "status", i32, 1, optional=True), _stream(stream)))


def moe_quantize_fp8(T: int, H: int, x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor,
                     flags: int = 0, stream=None) -> int:
    return _check("moe_quantize_fp8", _lib.moe_quantize_fp8(
        int(T), int(H), _dev(x, "x", _BF16_LIKE, T * H), _dev(q, "q", _FP8_CODES, T * H),
        _dev(scale, "scale", _fp8_scale_dtypes(flags), T * fp8_scale_cols(H, flags)),
        int(flags), _stream(stream)))


def moe_ll_layout_dispatch_fp8(shape: moe_shape, M: int, src_rank: int, topk_idx: torch.Tensor,
                               out: LayoutBuffers, x: torch.Tensor, recv_q: torch.Tensor,
                               recv_scale: torch.Tensor, recv_rows: int, flags: int = 0,
                               ws: Optional[torch.Tensor] = None, stream=None) -> int:
    T, H, K, E, R = shape.T, shape.H, shape.K, shape.E, shape.R
    idx = _dev(topk_idx, "topk_idx", (torch.int64,), T * K)
    st = out._struct(shape, int(M))
    wsp, wsn = _ws(ws, shape)
    return _check("moe_ll_layout_dispatch_fp8", _lib.moe_ll_layout_dispatch_fp8(
        C.byref(shape), int(M), int(src_rank), idx, C.byref(st), _dev(x, "x", _BF16_LIKE, T * H),
        _dev(recv_q, "recv_q", _FP8_CODES, int(recv_rows) * H),
        _dev(recv_scale, "recv_scale", _fp8_scale_dtypes(flags),
             _ll_scale_numel(E, R, M, H, recv_rows, flags)),
        int(recv_rows), int(flags), wsp, wsn, _stream(stream)))


def moe_ll_dispatch_fp8(shape: moe_shape, M: int, x: torch.Tensor, slot: torch.Tensor,
                        recv_q: torch.Tensor, recv_scale: torch.Tensor, recv_rows: int,
                        flags: int = 0, status: Optional[torch.Tensor] = None,
                        stream=None) -> int:
    T, H, K, E, R = shape.T, shape.H, shape.K, shape.E, shape.R
    return _check("moe_ll_dispatch_fp8", _lib.moe_ll_dispatch_fp8(
        C.byref(shape), int(M), _dev(x, "x", _BF16_LIKE, T * H),
        _dev(slot, "slot", (torch.int32,), T * K),
        _dev(recv_q, "recv_q", _FP8_CODES, int(recv_rows) * H),
        _dev(recv_scale, "recv_scale", _fp8_scale_dtypes(flags),
             _ll_scale_numel(E, R, M, H, recv_rows, flags)),
        int(recv_rows), int(flags), _dev(status, "status", (torch.int32,), 1, optional=True),
        _stream(stream)))


def moe_dispatch_fp8(shape: moe_shape, x_q: torch.Tensor, x_scale: torch.Tensor,
                     slot: torch.Tensor, recv_q: torch.Tensor, recv_scale: torch.Tensor,
                     recv_rows: int, status: Optional[torch.Tensor] = None, stream=None) -> int:
    T, H, K = shape.T, shape.H, shape.K
    G = H // FP8_GROUP
    return _check("moe_dispatch_fp8", _lib.moe_dispatch_fp8(
        C.byref(shape), _dev(x_q, "x_q", _FP8_CODES, T * H),
        _dev(x_scale, "x_scale", (torch.float32,), T * G),
        _dev(slot, "slot", (torch.int32,), T * K),
        _dev(recv_q, "recv_q", _FP8_CODES, int(recv_rows) * H),
        _dev(recv_scale, "recv_scale", (torch.float32,), int(recv_rows) * G), int(recv_rows),
        _dev(status, "status", (torch.int32,), 1, optional=True), _stream(stream)))


def moe_replica_weight_sync(E: int, E_phys: int, S: int, replica_count: torch.Tensor,
                            replica_phys: torch.Tensor, w: torch.Tensor,
                            status: Optional[torch.Tensor] = None, stream=None) -> int:
    i32 = (torch.int32,)
    return _check("moe_replica_weight_sync", _lib.moe_replica_weight_sync(
        int(E), int(E_phys), int(S), _dev(replica_count, "replica_count", i32, E),
        _dev(replica_phys, "replica_phys", i32, 2 * E), _dev(w, "w", _BF16_LIKE, E_phys * S),
        _dev(status, "status", i32, 1, optional=True), _stream(stream)))


def moe_replica_grad_reduce(E: int, E_phys: int, S: int, replica_count: torch.Tensor,
                            replica_phys: torch.Tensor, g: torch.Tensor,
                            status: Optional[torch.Tensor] = None, stream=None) -> int:
    i32 = (torch.int32,)
    return _check("moe_replica_grad_reduce", _lib.moe_replica_grad_reduce(
        int(E), int(E_phys), int(S), _dev(replica_count, "replica_count", i32, E),
        _dev(replica_phys, "replica_phys", i32, 2 * E),
        _dev(g, "g", (torch.float32,), E_phys * S),
        _dev(status, "status", i32, 1, optional=True), _stream(stream)))
