"""The other paths captured in HIP graphs (as the benchmark replays them):
every replay, with eager work and synchronisation between replays, gives the
eager outputs bit for bit. Covers the low-latency FP8 dispatch (both scale
layouts) with combine, the normal-mode path, the masked combine and the
replica route (load, plan, reroute, layout, dispatch, combine)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from gpu_path import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def capi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_moe_layout_03_amd import capi as c

    return c


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def replay_check(step, outputs, poison, reps=3):
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step(stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(stream)
    for rep in range(reps):
        for t in poison:
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, ref)):
            # bit patterns: rows a call leaves untouched may hold NaN
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                f"replay {rep}: output {i} differs"
        junk = torch.randn(1 << 20, device=dev()).sum()
        assert torch.isfinite(junk)
    return ref


@pytest.mark.parametrize("flags", [0, 3, 4])
def test_graph_low_latency_fp8(capi, orc, flags):
    M = 64
    w = mi.config_c3(M)
    E, R, K, T, H = w.E, w.R, w.K, w.T, w.H
    shape = capi.make_shape(T, H, E, R, K, 1)
    rows = E * R * M
    idx, x, wt = to_dev(w.topk_idx), to_dev(w.x), to_dev(w.topk_weights)
    lay = capi.LayoutBuffers.empty(shape, dev(), ll_M=M)
    cols = capi.fp8_scale_cols(H, flags)
    q = torch.zeros(rows, H, dtype=torch.uint8, device=dev())
    sshape = (rows, cols) if flags & 4 else (E, cols, R * M)
    sc = torch.zeros(sshape, dtype=torch.int32 if flags & 2 else torch.float32, device=dev())
    y = torch.zeros(rows, H, dtype=torch.int16, device=dev())
    out = torch.empty(T, H, dtype=torch.int16, device=dev())
    capi.moe_ll_layout_dispatch(shape, M, 2, idx, lay, x, y, rows)  # expert output stand-in
    torch.cuda.synchronize()
    _announce(f"graph: low-latency FP8 flags={flags} + combine")

    def step(s):
        capi.moe_ll_layout_dispatch_fp8(shape, M, 2, idx, lay, x, q, sc, rows, flags, stream=s)
        capi.moe_combine(shape, y, rows, lay.slot, wt, out, None, lay.status, stream=s)

    replay_check(step, [lay.count, lay.slot, q, sc, out], [lay.count, lay.slot, out])
    ll = orc.ll_layout(w.topk_idx, E, R, M, 2)
    assert np.array_equal(lay.slot.cpu().numpy().reshape(T, K), ll["slot"])


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "one_call"])
def test_graph_normal_mode(capi, orc, fused):
    w = mi.config_c2()
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    idx, x, wt = to_dev(w.topk_idx), to_dev(w.x), to_dev(w.topk_weights)
    lay = capi.RankLayoutBuffers.empty(shape, dev())
    recv = torch.zeros(max(lay.cap, 1), w.H, dtype=torch.int16, device=dev())
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev())
    ow = torch.empty(w.T, w.K, dtype=torch.float32, device=dev())
    _announce(f"graph: normal-mode layout + dispatch + combine, fused={fused}")

    def step(s):
        if fused:
            capi.moe_rank_layout_dispatch(shape, idx, wt, lay, x, recv, lay.cap, stream=s)
        else:
            capi.moe_rank_layout(shape, idx, wt, lay, stream=s)
            capi.moe_rank_dispatch(shape, x, lay.rank_slot, recv, lay.cap, lay.status, stream=s)
        capi.moe_rank_combine(shape, recv, lay.cap, lay.rank_slot, lay.recv_topk_weights, out,
                              None, ow, lay.status, stream=s)

    replay_check(step, [lay.rank_slot, lay.rank_offset, lay.recv_topk_idx,
                        lay.recv_topk_weights, recv, out, ow],
                 [lay.rank_slot, lay.rank_offset, out, ow])
    ref = orc.rank_layout(w.topk_idx, w.E, w.R, 1, w.topk_weights)
    assert np.array_equal(lay.rank_slot.cpu().numpy().reshape(w.T, w.R), ref["rank_slot"])


def test_graph_masked_combine(capi, orc):
    w = mi.config_c2()
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    lay_ref = orc.layout(w.topk_idx, w.E, w.R, 1)
    rows = lay_ref["rows"]
    y = to_dev(mi.to_bf16_bits(np.random.default_rng(3).standard_normal(
        (rows, w.H)).astype(np.float32)))
    slot = to_dev(lay_ref["slot"].astype(np.int32))
    idx, wt = to_dev(w.topk_idx), to_dev(w.topk_weights)
    mask = torch.zeros(w.R, dtype=torch.int32, device=dev())
    mask[3] = 1
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev())
    _announce("graph: masked combine")

    def step(s):
        capi.moe_combine_masked(shape, y, rows, slot, idx, wt, mask, out, None, None, stream=s)

    replay_check(step, [out], [out])


def test_graph_replica_route(capi, orc):
    w = mi.config_c5(T=2048, H=512)
    E, R, K, T, H, C = w.E, w.R, w.K, w.T, w.H, w.replicas
    Ep = E + C
    shape = capi.make_shape(T, H, Ep, R, K, 1)
    idx, x, wt = to_dev(w.topk_idx), to_dev(w.x), to_dev(w.topk_weights)
    i32 = dict(dtype=torch.int32, device=dev())
    load, rc = torch.empty(E, **i32), torch.empty(E, **i32)
    rp, p2l = torch.empty(E, 2, **i32), torch.empty(Ep, **i32)
    phys = torch.empty(T, K, dtype=torch.int64, device=dev())
    lay = capi.LayoutBuffers.empty(shape, dev())
    rows = capi.moe_recv_rows_worst(shape)
    recv = torch.zeros(rows, H, dtype=torch.int16, device=dev())
    out = torch.empty(T, H, dtype=torch.int16, device=dev())
    ws = torch.empty(max(capi.moe_layout_workspace_bytes(shape), 1), dtype=torch.uint8,
                     device=dev())
    _announce("graph: replica route (load, plan, reroute, layout+dispatch, combine)")

    def step(s):
        capi.moe_expert_load(T, K, E, idx, load, None, stream=s)
        capi.moe_plan_replicas(E, R, C, load, rc, rp, p2l, stream=s)
        capi.moe_reroute(T, K, E, idx, rc, rp, Ep, phys, None, stream=s)
        capi.moe_layout_dispatch(shape, phys, lay, x, recv, rows, ws, stream=s)
        capi.moe_combine(shape, recv, rows, lay.slot, wt, out, None, lay.status, stream=s)

    replay_check(step, [load, rc, rp, p2l, phys, lay.slot, lay.count, out],
                 [load, rc, phys, lay.slot, out])
    ref_load, _ = orc.expert_load(w.topk_idx, E)
    assert np.array_equal(load.cpu().numpy(), ref_load)


def test_graph_layout_dispatch_static(capi, orc):
    """moe_layout_dispatch_static, the entry point for callers that cannot
    allocate, captured in a graph at a size whose layout runs in three
    launches over the library's static per-GPU scratch: every replay equals
    the eager call, and that call equals the oracle."""
    w = mi.random_case(31, 1100, 256, 64, 8, 8, 1, neg_frac=0.02)  # 8800 pairs
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    assert capi.moe_layout_workspace_bytes(shape) > 0
    _announce(f"graph: static-scratch layout + dispatch, T={w.T} K={w.K}")
    idx, x = to_dev(w.topk_idx), to_dev(w.x)
    lay = capi.LayoutBuffers.empty(shape, dev())
    rows = capi.moe_recv_rows_worst(shape)
    recv = torch.full((rows, w.H), -7, dtype=torch.int16, device=dev())

    def step(s):
        capi.moe_layout_dispatch_static(shape, idx, lay, x, recv, rows, stream=s)

    # (row_src past the rows in use is never written, so it is compared but not poisoned)
    ref = replay_check(step, [lay.slot, lay.count, lay.offset, lay.row_src, recv],
                       [lay.slot, lay.count, lay.offset])
    o = orc.layout(w.topk_idx, w.E, w.R, 1)
    assert np.array_equal(ref[0].cpu().numpy().reshape(w.T, w.K), o["slot"])
    assert np.array_equal(ref[1].cpu().numpy(), o["count"])
    assert np.array_equal(ref[2].cpu().numpy(), o["offset"])
    r = o["rows"]
    rref, _ = orc.dispatch(w.x, o["slot"], r, fill=-7 & 0xFFFF)
    assert np.array_equal(ref[4].cpu().numpy()[:r].view(np.uint16), rref.view(np.uint16))
