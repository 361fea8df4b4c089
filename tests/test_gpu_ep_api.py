"""The page-named convenience calls (ep.py) end to end on the GPU, against the
oracle: get_dispatch_layout + dispatch + combine, dispatch of an FP8 tuple,
low_latency_dispatch (bf16 and FP8, with cumulative receive counts),
low_latency_combine (with an active-rank mask), and the normal-mode dispatch
(bf16 and an FP8 tuple) and combine."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from gpu_path import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_moe_layout_03_amd import ep as e

    return e


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_layout_dispatch_combine(ep, orc):
    w = mi.config_c1()
    idx = to_dev(w.topk_idx)
    x = to_dev(w.x).view(torch.bfloat16)
    rtc, none, cnt, in_rank, h = ep.get_dispatch_layout(idx, w.E, w.R, 4, w.H)
    ref = orc.layout(w.topk_idx, w.E, w.R, 4)
    assert none is None
    assert np.array_equal(cnt.cpu().numpy(), ref["count"])
    assert np.array_equal(rtc.cpu().numpy(), ref["rank_token_count"])
    assert np.array_equal(in_rank.cpu().numpy(), ref["is_token_in_rank"].astype(bool))
    recv = ep.dispatch(x, h)
    rref, _ = orc.dispatch(w.x, ref["slot"], ref["rows"], fill=0)
    used = np.zeros(ref["rows"], bool)
    used[ref["slot"][ref["slot"] >= 0]] = True
    assert np.array_equal(_bits(recv)[:ref["rows"]][used], rref[used])
    out = ep.combine(recv, h, to_dev(w.topk_weights))
    r32 = orc.combine(rref, ref["slot"], w.topk_weights, "f32")
    assert np.array_equal(_bits(out), r32["out_bf16"])


def test_dispatch_fp8_tuple(ep, orc):
    w = mi.config_c2()
    idx = to_dev(w.topk_idx)
    qz = orc.quantize_fp8(w.x, 0)
    _, _, _, _, h = ep.get_dispatch_layout(idx, w.E, w.R, 1, w.H)
    xq = torch.from_numpy(qz["q"]).to(dev()).view(torch.float8_e4m3fn)
    rq, rs = ep.dispatch((xq, to_dev(qz["scale"])), h)
    ref = orc.layout(w.topk_idx, w.E, w.R, 1)
    wq, ws_, _ = orc.dispatch_fp8_tuple(qz["q"], qz["scale"], ref["slot"], ref["rows"])
    assert np.array_equal(rq.view(torch.uint8).cpu().numpy()[:ref["rows"]], wq)
    assert np.array_equal(rs.cpu().numpy()[:ref["rows"]].view(np.uint32),
                          ws_.view(np.uint32))


@pytest.mark.parametrize("use_fp8,round_scale,use_ue8m0,scale_rows",
                         [(False, False, False, False), (True, False, False, False),
                          (True, True, True, False), (True, False, False, True)])
def test_low_latency_dispatch_and_masked_combine(ep, orc, use_fp8, round_scale, use_ue8m0,
                                                  scale_rows):
    M, src = 64, 3
    w = mi.config_c3(M)
    E, R, K, H, L = w.E, w.R, w.K, w.H, w.E // w.R
    idx = to_dev(w.topk_idx)
    x = to_dev(w.x).view(torch.bfloat16)
    stats = torch.full((E,), 10, dtype=torch.int32, device=dev())
    recv, cnt, h = ep.low_latency_dispatch(x, idx, M, E, R, src,
                                           cumulative_local_expert_recv_stats=stats,
                                           use_fp8=use_fp8, round_scale=round_scale,
                                           use_ue8m0=use_ue8m0, scale_rows=scale_rows)
    ll = orc.ll_layout(w.topk_idx, E, R, M, src)
    # the low-latency handle carries no normal-path rank tables
    assert h.layout.rank_token_count is None and h.layout.is_token_in_rank is None
    assert np.array_equal(h.layout.row_src.cpu().numpy(), ll["row_src"])
    assert np.array_equal(cnt.cpu().numpy(), ll["recv_count"])
    assert np.array_equal(stats.cpu().numpy(), 10 + ll["recv_count"])
    rows = E * R * M
    v = ll["slot"] >= 0
    tok = np.repeat(np.arange(w.T), K).reshape(w.T, K)[v]
    sl = ll["slot"][v]
    if use_fp8:
        flags = (1 if round_scale or use_ue8m0 else 0) | (2 if use_ue8m0 else 0)
        q, sc = recv
        assert q.shape == (R, L, R * M, H)
        qz = orc.quantize_fp8(w.x, flags)
        qn = q.reshape(rows, H).view(torch.uint8).cpu().numpy()
        assert np.array_equal(qn[sl], qz["q"][tok])
        cols = H // 512 if use_ue8m0 else H // 128
        assert sc.shape == (R, L, R * M, cols)
        sn = sc.reshape(rows, cols).cpu().numpy()  # page view: [.., R*M, cols]
        want = (qz["ue8m0"] if use_ue8m0 else qz["scale"])[tok]
        assert np.array_equal(sn[sl].view(np.uint32), want.view(np.uint32))
        return
    assert recv.shape == (R, L, R * M, H)
    flat = recv.reshape(rows, H)
    assert np.array_equal(_bits(flat[torch.from_numpy(sl).to(dev())]), w.x[tok])
    # low_latency_combine with ranks 0 and 6 masked
    mask = np.zeros(R, np.int32)
    mask[[0, 6]] = 1
    out = ep.low_latency_combine(recv, to_dev(w.topk_weights), h, rank_mask=to_dev(mask))
    y = np.zeros((rows, H), np.uint16)
    y[sl] = w.x[tok]
    ref = orc.combine_masked(y, ll["slot"], w.topk_idx, E, R, mask, w.topk_weights)
    assert np.array_equal(_bits(out), ref["out_bf16"])
    out2 = ep.low_latency_combine(recv, to_dev(w.topk_weights), h)
    assert np.array_equal(_bits(out2), orc.combine(y, ll["slot"], w.topk_weights,
                                                   "f32")["out_bf16"])


def test_normal_dispatch_and_combine(ep, orc):
    w = mi.config_c2()
    x = to_dev(w.x).view(torch.bfloat16)
    recv, ridx, rw, rcount, roff, h = ep.normal_dispatch(x, to_dev(w.topk_idx),
                                                         to_dev(w.topk_weights), w.E, w.R, 4)
    ref = orc.rank_layout(w.topk_idx, w.E, w.R, 4, w.topk_weights)
    rows = ref["rows"]
    assert np.array_equal(roff.cpu().numpy(), ref["rank_offset"])
    assert np.array_equal(rcount.cpu().numpy(), ref["recv_expert_count"])
    assert np.array_equal(ridx.cpu().numpy()[:rows], ref["recv_topk_idx"])
    assert np.array_equal(rw.cpu().numpy()[:rows], ref["recv_topk_weights"])
    assert np.array_equal(_bits(recv)[:rows], w.x[ref["recv_src"]])
    out, cw = ep.normal_combine(recv, h, rw)
    rref, _ = orc.dispatch(w.x, ref["rank_slot"], max(w.T * min(w.K, w.R), 1), fill=0)
    assert np.array_equal(_bits(out), orc.combine(rref, ref["rank_slot"], None,
                                                  "f32")["out_bf16"])
    want, _ = orc.combine_rank_weights(ref["rank_slot"], ref["recv_topk_weights"])
    assert np.array_equal(cw.cpu().numpy(), want)


def test_normal_dispatch_fp8_tuple(ep, orc):
    """Normal mode with x given as an (E4M3, scales) tuple: the rank rows
    receive each token's codes and scales bit for bit."""
    w = mi.config_c2()
    qz = orc.quantize_fp8(w.x, 0)
    xq = torch.from_numpy(qz["q"]).to(dev()).view(torch.float8_e4m3fn)
    (rq, rs), ridx, rw, rcount, roff, h = ep.normal_dispatch(
        (xq, to_dev(qz["scale"])), to_dev(w.topk_idx), to_dev(w.topk_weights), w.E, w.R, 1)
    ref = orc.rank_layout(w.topk_idx, w.E, w.R, 1, w.topk_weights)
    rows = ref["rows"]
    assert np.array_equal(roff.cpu().numpy(), ref["rank_offset"])
    assert np.array_equal(ridx.cpu().numpy()[:rows], ref["recv_topk_idx"])
    wq, ws_, st = orc.dispatch_fp8_tuple(qz["q"], qz["scale"], ref["rank_slot"],
                                         max(w.T * min(w.K, w.R), 1))
    assert st == 0
    assert np.array_equal(rq.view(torch.uint8).cpu().numpy()[:rows], wq[:rows])
    assert np.array_equal(rs.cpu().numpy()[:rows].view(np.uint32), ws_[:rows].view(np.uint32))
    assert np.array_equal(rq.view(torch.uint8).cpu().numpy()[:rows], qz["q"][ref["recv_src"]])
