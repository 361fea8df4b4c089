"""Parity with the oracle of the combine with an active-rank mask and of the
cumulative per-expert receive counts (Buffer.low_latency_dispatch,
cumulative_local_expert_recv_stats).

Bar: the masked combine bit-exact against the oracle's float ascending-k sum
(and within 1e-2 rel + 1e-3 abs of the dense f64 sum); receive counts exact.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from gpu_path import dev, np16, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def capi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_moe_layout_03_amd import capi as c

    return c


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_masked_combine(capi, w, slot, rows, y, mask, weights=True):
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    out = torch.full((w.T, w.H), 0x1234, dtype=torch.int16, device=dev())
    o32 = torch.full((w.T, w.H), float("nan"), dtype=torch.float32, device=dev())
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    capi.moe_combine_masked(shape, to_dev(y), rows, to_dev(slot.astype(np.int32)),
                            to_dev(w.topk_idx.astype(np.int64)),
                            to_dev(w.topk_weights) if weights else None,
                            to_dev(mask.astype(np.int32)), out, o32, st)
    torch.cuda.synchronize()
    return np16(out), o32.cpu().numpy(), int(st.item())


def check_masked(capi, orc, w, slot, rows, y, mask, weights=True):
    g16, g32, st = gpu_masked_combine(capi, w, slot, rows, y, mask, weights)
    ref = orc.combine_masked(y, slot, w.topk_idx, w.E, w.R, mask,
                             w.topk_weights if weights else None)
    assert st == ref["status"]
    assert np.array_equal(g16, ref["out_bf16"]), "bf16 out"
    assert np.array_equal(g32.view(np.uint32), ref["out_f32"].view(np.uint32)), "f32 out"
    # the stated tolerance against the exact sum, through the dense form
    L = w.E // w.R
    s2 = np.where((w.topk_idx >= 0) & (w.topk_idx < w.E)
                  & (mask[np.clip(w.topk_idx, 0, w.E - 1) // L] != 0), -1, slot)
    r64 = orc.combine(y, s2, w.topk_weights if weights else None, "f64")["out_f64"]
    g = mi.bf16_bits_to_f32(g16).astype(np.float64)
    assert np.all(np.abs(g - r64) <= 1e-3 + 1e-2 * np.abs(r64))


CASES = [
    # (seed, T, H, E, R, K, neg, dup)
    (1, 33, 72, 16, 4, 3, 0.1, 0.2),
    (2, 100, 256, 64, 8, 6, 0.0, 0.0),
    (3, 7, 1032, 8, 2, 8, 0.3, 0.3),
    (4, 1, 8, 4, 4, 1, 0.0, 0.0),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("ll", [False, True])
def test_masked_combine_random(capi, orc, case, ll):
    seed, T, H, E, R, K, neg, dup = case
    w = mi.random_case(1100 + seed, T, H, E, R, K, 1, neg_frac=neg, dup_frac=dup)
    rng = np.random.default_rng(seed)
    if ll:
        M = T
        lay = orc.ll_layout(w.topk_idx, E, R, M, R - 1)
        rows = E * R * M
    else:
        lay = orc.layout(w.topk_idx, E, R, 1)
        rows = max(lay["rows"], 1)
    y = mi.to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    for mask in (rng.random(R) < 0.4, np.zeros(R, bool), np.ones(R, bool)):
        _announce(f"masked combine seed={seed} ll={ll} mask={mask.astype(int).tolist()}")
        check_masked(capi, orc, w, lay["slot"], rows, y, mask.astype(np.int32))
    check_masked(capi, orc, w, lay["slot"], rows, y, (rng.random(R) < 0.5).astype(np.int32),
                 weights=False)


def test_masked_combine_standard_and_low_latency(capi, orc):
    """128 x 7168, 256 experts top-8: ranks 1 and 5 masked, contiguous layout
    (identity expert: y = the dispatched rows) and low-latency layout."""
    w = mi.config_c2()
    mask = np.zeros(w.R, np.int32)
    mask[[1, 5]] = 1
    lay = orc.layout(w.topk_idx, w.E, w.R, 1)
    recv, _ = orc.dispatch(w.x, lay["slot"], lay["rows"], fill=0)
    _announce("masked combine 128x7168 contiguous")
    check_masked(capi, orc, w, lay["slot"], lay["rows"], recv, mask)
    w3 = mi.config_c3(128)
    ll = orc.ll_layout(w3.topk_idx, w3.E, w3.R, 128, 2)
    rows = w3.E * w3.R * 128
    # only the written stripe matters; untouched rows are never read
    y = np.zeros((rows, w3.H), np.uint16)
    v = ll["slot"] >= 0
    t_idx = np.repeat(np.arange(w3.T), w3.K).reshape(w3.T, w3.K)
    y[ll["slot"][v]] = w3.x[t_idx[v]]
    _announce("masked combine 128x7168 low latency")
    check_masked(capi, orc, w3, ll["slot"], rows, y, mask)


def test_masked_combine_bad_slot_on_masked_rank_not_reported(capi, orc):
    w = mi.random_case(1120, 20, 64, 16, 4, 2, 1)
    lay = orc.layout(w.topk_idx, 16, 4, 1)
    slot = lay["slot"].copy()
    e0 = int(w.topk_idx[3, 0])
    slot[3, 0] = 10 ** 6  # out of range, on rank e0 // 4
    y = mi.to_bf16_bits(np.random.default_rng(5).standard_normal((lay["rows"], 64)).astype(
        np.float32))
    mask = np.zeros(4, np.int32)
    mask[e0 // 4] = 1
    _announce("masked combine: bad slot on a masked rank")
    g16, g32, st = gpu_masked_combine(capi, w, slot, lay["rows"], y, mask)
    assert st == 0
    mask[:] = 0
    g16, g32, st = gpu_masked_combine(capi, w, slot, lay["rows"], y, mask)
    assert st == 4


def _stats_run(capi, w, ll, M, src, times, init, fused):
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    lay = capi.LayoutBuffers.empty(shape, dev(), ll_M=M if ll else None)
    lay.recv_stats = to_dev(init.astype(np.int32))
    nws = capi.moe_layout_workspace_bytes(shape)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev()) if nws else None
    idx = to_dev(w.topk_idx.astype(np.int64))
    for _ in range(times):
        if fused:
            rows = w.E * w.R * M if ll else capi.moe_recv_rows_worst(shape)
            recv = torch.empty((rows, w.H), dtype=torch.int16, device=dev())
            x = to_dev(w.x)
            if ll:
                capi.moe_ll_layout_dispatch(shape, M, src, idx, lay, x, recv, rows, ws)
            else:
                capi.moe_layout_dispatch(shape, idx, lay, x, recv, rows, ws)
        elif ll:
            capi.moe_ll_layout(shape, M, src, idx, lay, ws)
        else:
            capi.moe_layout(shape, idx, lay, ws)
    torch.cuda.synchronize()
    return lay.recv_stats.cpu().numpy()


STATS_CASES = [
    # (name, T, K, E, R, ll)  -> fused count kernel / one-block / multi-block layouts
    ("fused_ll", 64, 8, 64, 8, True),
    ("fused_contig", 64, 8, 64, 8, False),
    ("oneblock_ll", 600, 8, 64, 8, True),
    ("oneblock_contig", 600, 8, 64, 8, False),
    ("multiblock_ll", 2000, 8, 128, 8, True),
    ("multiblock_contig", 3000, 6, 96, 4, False),
]


@pytest.mark.parametrize("case", STATS_CASES, ids=[c[0] for c in STATS_CASES])
@pytest.mark.parametrize("fused", [True, False])
def test_recv_stats(capi, orc, case, fused):
    name, T, K, E, R, ll = case
    w = mi.random_case(1200 + T, T, 64, E, R, K, 1, neg_frac=0.05, dup_frac=0.05)
    M = T
    init = np.arange(E, dtype=np.int32) * 3 - 7
    _announce(f"recv stats {name} fused={fused}")
    got = _stats_run(capi, w, ll, M, R - 1, 3, init, fused)
    if ll:
        cnt = orc.ll_layout(w.topk_idx, E, R, M, R - 1)["recv_count"]
    else:
        cnt = orc.layout(w.topk_idx, E, R, 1)["count"]
    want = init.copy()
    for _ in range(3):
        want = orc.accumulate_recv_stats(cnt, want)
    assert np.array_equal(got, want)
