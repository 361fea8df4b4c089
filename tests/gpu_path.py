"""Helpers for the GPU tests: run the HIP path through the C ABI on a
Workload and bring results back as numpy. Nothing here computes expected
values; those come from the oracle only."""
from __future__ import annotations

import numpy as np
import torch

SENTINEL = 0x7E57  # bf16 pattern pre-filled into receive buffers


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def np16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run_layout(capi, w, A=None, ll=False, M=None, src=0, idx=None, E=None, extras=True):
    """Layout on the GPU; returns (numpy dict, LayoutBuffers, shape)."""
    idx_np = w.topk_idx if idx is None else idx
    E = w.E if E is None else E
    A = w.A if A is None else A
    shape = capi.make_shape(w.T, w.H, E, w.R, w.K, A)
    d_idx = to_dev(idx_np.astype(np.int64))
    if ll:
        lay = capi.LayoutBuffers.empty(shape, dev(), ll_M=M, extras=extras)
    else:
        lay = capi.LayoutBuffers.empty(shape, dev(), extras=extras)
    # poison the outputs: nothing may rely on zero-initialised buffers
    for t in (lay.count, lay.offset, lay.slot, lay.rank_token_count, lay.row_src):
        if t is not None:
            t.fill_(-12345)
    if lay.is_token_in_rank is not None:
        lay.is_token_in_rank.fill_(7)
    nws = capi.moe_layout_workspace_bytes(shape)
    ws = torch.full((max(nws, 1),), 0xA5, dtype=torch.uint8, device=dev()) if nws else None
    if ll:
        capi.moe_ll_layout(shape, M, src, d_idx, lay, ws)
    else:
        capi.moe_layout(shape, d_idx, lay, ws)
    torch.cuda.synchronize()
    out = dict(count=lay.count.cpu().numpy(), slot=lay.slot.cpu().numpy().reshape(w.T, w.K),
               status=int(lay.status.item()))
    if not ll:
        out["offset"] = lay.offset.cpu().numpy()
        out["rows"] = int(out["offset"][E])
    else:
        out["offset"] = lay.offset.cpu().numpy()
        out["rows"] = E * w.R * M
    if extras:
        out["rank_token_count"] = lay.rank_token_count.cpu().numpy()
        out["is_token_in_rank"] = lay.is_token_in_rank.cpu().numpy().reshape(w.T, w.R)
        rs = lay.row_src.cpu().numpy()
        out["row_src"] = rs[: E * M] if ll else rs[: out["rows"]]
    return out, lay, shape


def run_dispatch_combine(capi, w, shape, lay, rows, weights=True, f32=True, x=None,
                         recv_fill=SENTINEL, y=None):
    """Dispatch into a sentinel-filled buffer, then combine (identity expert
    unless y is given). Returns numpy recv, out_bf16, out_f32, status."""
    x_np = w.x if x is None else x
    d_x = to_dev(x_np)
    recv = torch.full((max(rows, 1), w.H), recv_fill - 65536 if recv_fill > 32767 else recv_fill,
                      dtype=torch.int16, device=dev())
    capi.moe_dispatch(shape, d_x, lay.slot, recv, rows, lay.status)
    src = recv if y is None else to_dev(y)
    out = torch.full((w.T, w.H), 0x1234, dtype=torch.int16, device=dev())
    o32 = torch.full((w.T, w.H), float("nan"), dtype=torch.float32, device=dev()) if f32 else None
    wt = to_dev(w.topk_weights) if weights else None
    capi.moe_combine(shape, src, rows, lay.slot, wt, out, o32, lay.status)
    torch.cuda.synchronize()
    return (np16(recv), np16(out), o32.cpu().numpy() if f32 else None,
            int(lay.status.item()))


def run_layout_dispatch(capi, w, A=None, ll=False, M=None, src=0, rows=None):
    """moe_layout_dispatch / moe_ll_layout_dispatch on the GPU into a
    sentinel-filled receive buffer; returns (layout dict, recv numpy, lay, shape)."""
    A = w.A if A is None else A
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, A)
    d_idx = to_dev(w.topk_idx.astype(np.int64))
    lay = capi.LayoutBuffers.empty(shape, dev(), ll_M=M if ll else None)
    for t in (lay.count, lay.offset, lay.slot, lay.rank_token_count, lay.row_src):
        t.fill_(-12345)
    lay.is_token_in_rank.fill_(7)
    if rows is None:
        rows = capi.moe_ll_recv_rows(w.E, w.R, M) if ll else capi.moe_recv_rows_worst(shape)
    recv = torch.full((max(rows, 1), w.H), SENTINEL, dtype=torch.int16, device=dev())
    nws = capi.moe_layout_workspace_bytes(shape)
    ws = torch.full((max(nws, 1),), 0x5A, dtype=torch.uint8, device=dev()) if nws else None
    x = to_dev(w.x)
    if ll:
        capi.moe_ll_layout_dispatch(shape, M, src, d_idx, lay, x, recv, rows, ws)
    else:
        capi.moe_layout_dispatch(shape, d_idx, lay, x, recv, rows, ws)
    torch.cuda.synchronize()
    E = w.E
    out = dict(count=lay.count.cpu().numpy(), slot=lay.slot.cpu().numpy().reshape(w.T, w.K),
               status=int(lay.status.item()), offset=lay.offset.cpu().numpy(),
               rank_token_count=lay.rank_token_count.cpu().numpy(),
               is_token_in_rank=lay.is_token_in_rank.cpu().numpy().reshape(w.T, w.R))
    rs = lay.row_src.cpu().numpy()
    out["rows"] = E * w.R * M if ll else int(out["offset"][E])
    out["row_src"] = rs[: E * M] if ll else rs[: out["rows"]]
    return out, recv, lay, shape
