"""Allocating convenience layer with the expert-parallel buffer's call names.

The names and return tuples mirror the NeMo AutoModel page
"nemo_automodel.components.moe.uccl_ep.buffer" (Buffer.get_dispatch_layout,
Buffer.dispatch, Buffer.combine, Buffer.low_latency_dispatch,
Buffer.low_latency_combine) reduced to one GPU: the R logical ranks are
partitions of one HBM receive buffer and nothing crosses a GPU boundary. The
replica calls mirror the "dots-infra/ultraep architecture" page (Load
computation, Placement planning, Routing expansion).

This layer only allocates torch tensors and calls the C ABI through ``capi``;
every step runs in the library's kernels, on the current torch stream, with
no host synchronisation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple, Union

import torch

from . import capi


@dataclass
class Handle:
    """What dispatch hands on to combine: the shape and the layout arrays."""

    shape: capi.moe_shape
    layout: capi.LayoutBuffers
    recv_rows: int
    ll_M: Optional[int] = None
    src_rank: int = 0
    topk_idx: Optional[torch.Tensor] = None  # kept for a masked combine


def _workspace(shape: capi.moe_shape, device) -> Optional[torch.Tensor]:
    n = capi.moe_layout_workspace_bytes(shape)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                        expert_alignment: int = 1, hidden: int = 8):
    """Returns (num_tokens_per_rank [R] int32, None, num_tokens_per_expert [E] int32,
    is_token_in_rank [T, R] bool, handle). The per-RDMA-rank counts are None,
    as for a single node."""
    T, K = topk_idx.shape
    shape = capi.make_shape(T, hidden, num_experts, num_ranks, K, expert_alignment)
    lay = capi.LayoutBuffers.empty(shape, topk_idx.device)
    capi.moe_layout(shape, topk_idx.contiguous(), lay, _workspace(shape, topk_idx.device))
    h = Handle(shape, lay, capi.moe_recv_rows_worst(shape))
    return (lay.rank_token_count, None, lay.count,
            lay.is_token_in_rank.view(T, num_ranks).bool(), h)


def dispatch(x: Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]], handle: Handle,
             recv_x: Optional[torch.Tensor] = None):
    """Scatter rows into the contiguous receive buffer, sized for the worst
    case (T*K + E*(A-1) rows, so no host read of the counts is needed).
    Rows [offset[e], offset[e] + count[e]) belong to expert e. x is bf16
    [T, H], or (as on the page) a tuple of E4M3 codes [T, H] and float scales
    [T, H/128], in which case the result is the tuple (codes, scales) of the
    receive rows."""
    if isinstance(x, tuple):
        xq, xs = x
        T, H = xq.shape
        shape = capi.make_shape(T, H, handle.shape.E, handle.shape.R, handle.shape.K,
                                handle.shape.A)
        handle.shape = shape
        rows = max(handle.recv_rows, 1)
        rq = torch.empty(rows, H, dtype=xq.dtype, device=xq.device)
        rs = torch.empty(rows, H // capi.FP8_GROUP, dtype=torch.float32, device=xq.device)
        capi.moe_dispatch_fp8(shape, xq.contiguous(), xs.contiguous(), handle.layout.slot,
                              rq.view(torch.uint8), rs, handle.recv_rows, handle.layout.status)
        return rq, rs
    T, H = x.shape
    shape = capi.make_shape(T, H, handle.shape.E, handle.shape.R, handle.shape.K,
                            handle.shape.A)
    handle.shape = shape
    if recv_x is None:
        recv_x = torch.empty(max(handle.recv_rows, 1), H, dtype=x.dtype, device=x.device)
    capi.moe_dispatch(shape, x.contiguous(), handle.layout.slot, recv_x, handle.recv_rows,
                      handle.layout.status)
    return recv_x


def dispatch_with_layout(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int,
                         num_ranks: int, expert_alignment: int = 1,
                         recv_x: Optional[torch.Tensor] = None):
    """Layout and dispatch in one call (Buffer.dispatch given topk_idx and no
    handle). Returns (recv_x, handle); the handle carries the layout arrays."""
    T, H = x.shape
    K = topk_idx.shape[1]
    shape = capi.make_shape(T, H, num_experts, num_ranks, K, expert_alignment)
    lay = capi.LayoutBuffers.empty(shape, x.device)
    rows = capi.moe_recv_rows_worst(shape)
    if recv_x is None:
        recv_x = torch.empty(max(rows, 1), H, dtype=x.dtype, device=x.device)
    capi.moe_layout_dispatch(shape, topk_idx.contiguous(), lay, x.contiguous(), recv_x, rows,
                             _workspace(shape, x.device))
    return recv_x, Handle(shape, lay, rows)


def combine(y: torch.Tensor, handle: Handle, topk_weights: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, out_f32: Optional[torch.Tensor] = None):
    """Weighted reduce of the expert outputs back to [T, H] bf16 (weights None:
    plain sum)."""
    shape = handle.shape
    H = y.shape[-1]
    if out is None:
        out = torch.empty(shape.T, H, dtype=torch.bfloat16, device=y.device)
    w = topk_weights.contiguous() if topk_weights is not None else None
    capi.moe_combine(shape, y.contiguous(), handle.recv_rows, handle.layout.slot, w, out,
                     out_f32, handle.layout.status)
    return out


def low_latency_dispatch(x: torch.Tensor, topk_idx: torch.Tensor,
                         num_max_dispatch_tokens_per_rank: int, num_experts: int,
                         num_ranks: int, src_rank: int = 0,
                         cumulative_local_expert_recv_stats: Optional[torch.Tensor] = None,
                         use_fp8: bool = False, round_scale: bool = False,
                         use_ue8m0: bool = False, scale_rows: bool = False,
                         recv_x: Optional[torch.Tensor] = None):
    """Padded low-latency dispatch from source rank ``src_rank``. Returns
    (recv_x [R, L, R*M, H] -- rank r's receive buffer is recv_x[r] --,
    recv_count [E] int32, handle). Only the source's stripe is written; rows
    past recv_count are not valid.

    use_fp8: recv_x is the tuple (E4M3 codes [R, L, R*M, H], scales), the
    scales as on the page: float [R, L, R*M, H/128] (UE8M0: int32
    [R, L, R*M, H/512]) whose last two dimensions are column-major; with
    scale_rows (an option of this library) they are row-major instead.
    cumulative_local_expert_recv_stats: an [E] int32 tensor (the R ranks'
    [L] tensors end to end) to which the receive counts are added."""
    T, H = x.shape
    K = topk_idx.shape[1]
    M = int(num_max_dispatch_tokens_per_rank)
    E, R = num_experts, num_ranks
    L = E // R
    shape = capi.make_shape(T, H, E, R, K, 1)
    # the low-latency handle: counts, slots, stripe offsets and source table
    # (no per-rank token counts or token-rank table, as on the page)
    lay = capi.LayoutBuffers.empty(shape, x.device, ll_M=M, rank_tables=False)
    lay.recv_stats = cumulative_local_expert_recv_stats
    rows = capi.moe_ll_recv_rows(E, R, M)
    ws = _workspace(shape, x.device)
    idx = topk_idx.contiguous()
    h = Handle(shape, lay, rows, ll_M=M, src_rank=src_rank, topk_idx=idx)
    if use_fp8:
        flags = ((capi.MOE_FP8_ROUND_SCALE if round_scale or use_ue8m0 else 0)
                 | (capi.MOE_FP8_UE8M0 if use_ue8m0 else 0)
                 | (capi.MOE_FP8_SCALE_ROWS if scale_rows else 0))
        cols = capi.fp8_scale_cols(H, flags)
        sdt = torch.int32 if use_ue8m0 else torch.float32
        q = torch.empty(rows, H, dtype=torch.float8_e4m3fn, device=x.device)
        if scale_rows:
            sc = torch.empty(rows, cols, dtype=sdt, device=x.device)
            sc_view = sc.view(R, L, R * M, cols)
        else:
            sc = torch.empty(E, cols, R * M, dtype=sdt, device=x.device)
            sc_view = sc.view(R, L, cols, R * M).transpose(2, 3)
        capi.moe_ll_layout_dispatch_fp8(shape, M, src_rank, idx, lay, x.contiguous(),
                                        q.view(torch.uint8), sc, rows, flags, ws)
        return (q.view(R, L, R * M, H), sc_view), lay.count, h
    if recv_x is None:
        recv_x = torch.empty(rows, H, dtype=x.dtype, device=x.device)
    capi.moe_ll_layout_dispatch(shape, M, src_rank, idx, lay, x.contiguous(), recv_x, rows, ws)
    return recv_x.view(R, L, R * M, H), lay.count, h


def low_latency_combine(y: torch.Tensor, topk_weights: torch.Tensor, handle: Handle,
                        out: Optional[torch.Tensor] = None,
                        rank_mask: Optional[torch.Tensor] = None):
    """Weighted reduce from the padded layout in place (the expert wrote its
    outputs straight into the padded buffer, as with zero_copy). rank_mask
    ([R] int32, nonzero = masked): pairs whose expert lives on a masked rank
    are left out (the combine's active-rank mask)."""
    if rank_mask is None:
        return combine(y.reshape(-1, y.shape[-1]), handle, topk_weights, out)
    shape = handle.shape
    H = y.shape[-1]
    if out is None:
        out = torch.empty(shape.T, H, dtype=torch.bfloat16, device=y.device)
    capi.moe_combine_masked(shape, y.reshape(-1, H).contiguous(), handle.recv_rows,
                            handle.layout.slot, handle.topk_idx, topk_weights.contiguous(),
                            rank_mask.contiguous(), out, None, handle.layout.status)
    return out


@dataclass
class RankHandle:
    """What normal-mode dispatch hands on to combine."""

    shape: capi.moe_shape
    layout: capi.RankLayoutBuffers
    recv_rows: int


def normal_dispatch(x: Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]],
                    topk_idx: torch.Tensor, topk_weights: Optional[torch.Tensor],
                    num_experts: int, num_ranks: int, expert_alignment: int = 1):
    """Buffer.dispatch in normal mode: each token is sent once to every rank
    hosting one of its experts. Returns (recv_x [rows, H], recv_topk_idx
    [rows, K] rank-local ids or -1, recv_topk_weights [rows, K] or None,
    num_recv_tokens_per_expert [E] int32 aligned to expert_alignment,
    rank_offset [R+1] int32, handle). The receive buffers of the R ranks are
    one buffer sized for the worst case, T * min(K, R) rows; rank r's tokens
    are rows [rank_offset[r], rank_offset[r+1]) (device values, no host
    read). x is bf16 [T, H], or (as on the page) a tuple of E4M3 codes
    [T, H] and float scales [T, H/128]; then recv_x is the tuple of the
    receive rows' codes and scales, each copied row for row."""
    fp8 = isinstance(x, tuple)
    xt = x[0] if fp8 else x
    T, H = xt.shape
    K = topk_idx.shape[1]
    shape = capi.make_shape(T, H, num_experts, num_ranks, K, expert_alignment)
    lay = capi.RankLayoutBuffers.empty(shape, xt.device, weights=topk_weights is not None)
    rows = max(lay.cap, 1)
    idx = topk_idx.contiguous()
    wts = topk_weights.contiguous() if topk_weights is not None else None
    if fp8:
        # the layout, then the tuple's row copy over the [T, R] table of rank rows
        xq, xs = x
        capi.moe_rank_layout(shape, idx, wts, lay)
        rq = torch.empty(rows, H, dtype=xq.dtype, device=xq.device)
        rs = torch.empty(rows, H // capi.FP8_GROUP, dtype=torch.float32, device=xq.device)
        rank_shape = capi.make_shape(T, H, num_experts, num_ranks, num_ranks, expert_alignment)
        capi.moe_dispatch_fp8(rank_shape, xq.contiguous(), xs.contiguous(), lay.rank_slot,
                              rq.view(torch.uint8), rs, lay.cap, lay.status)
        recv_x = (rq, rs)
    else:
        recv_x = torch.empty(rows, H, dtype=xt.dtype, device=xt.device)
        # layout and row copies in one call (one launch for batches of up to 1024 tokens)
        capi.moe_rank_layout_dispatch(shape, idx, wts, lay, xt.contiguous(), recv_x, lay.cap)
    w = lay.recv_topk_weights.view(rows, K) if lay.recv_topk_weights is not None else None
    return (recv_x, lay.recv_topk_idx.view(rows, K), w, lay.recv_expert_count,
            lay.rank_offset, RankHandle(shape, lay, lay.cap))


def normal_combine(y: torch.Tensor, handle: RankHandle,
                   topk_weights: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None):
    """Buffer.combine in normal mode: adds each token's rows back from the
    ranks it reached, without weights. Returns (combined_x [T, H] bf16,
    combined_topk_weights [T, K] or None -- the received weights summed back)."""
    shape = handle.shape
    H = y.shape[-1]
    if out is None:
        out = torch.empty(shape.T, H, dtype=torch.bfloat16, device=y.device)
    ow = None
    if topk_weights is not None:
        ow = torch.empty(shape.T, shape.K, dtype=torch.float32, device=y.device)
    capi.moe_rank_combine(shape, y.contiguous(), handle.recv_rows, handle.layout.rank_slot,
                          topk_weights.contiguous() if topk_weights is not None else None, out,
                          None, ow, handle.layout.status)
    return out, ow


def expert_load(topk_idx: torch.Tensor, num_experts: int,
                status: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, K = topk_idx.shape
    load = torch.empty(num_experts, dtype=torch.int32, device=topk_idx.device)
    capi.moe_expert_load(T, K, num_experts, topk_idx.contiguous(), load, status)
    return load


@dataclass
class ReplicaPlan:
    replica_count: torch.Tensor    # [E] 1 or 2
    replica_phys: torch.Tensor     # [E, 2] primary, replica or -1
    phys_to_logical: torch.Tensor  # [E + C]
    num_physical: int
    num_ranks: int


def plan_replicas(load: torch.Tensor, num_ranks: int, num_replicas: int) -> ReplicaPlan:
    E = load.numel()
    dev = load.device
    rc = torch.empty(E, dtype=torch.int32, device=dev)
    rp = torch.empty(E, 2, dtype=torch.int32, device=dev)
    p2l = torch.empty(E + num_replicas, dtype=torch.int32, device=dev)
    capi.moe_plan_replicas(E, num_ranks, num_replicas, load.contiguous(), rc, rp, p2l)
    return ReplicaPlan(rc, rp, p2l, E + num_replicas, num_ranks)


def reroute(topk_idx: torch.Tensor, plan: ReplicaPlan,
            status: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, K = topk_idx.shape
    E = plan.replica_count.numel()
    phys = torch.empty(T, K, dtype=torch.int64, device=topk_idx.device)
    capi.moe_reroute(T, K, E, topk_idx.contiguous(), plan.replica_count, plan.replica_phys,
                     plan.num_physical, phys, status)
    return phys
