"""Parity of the FP8 dispatch (through the C ABI) with the oracle.

Bar: bit-exact. The cast is an integer decision taken in the same precision
on both sides (float amax, float scale, correctly rounded float division,
round-to-nearest-even to E4M3), so every code byte, every float scale and
every UE8M0 word must match the oracle exactly; rows and scale entries no pair
maps to must keep their sentinel.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from gpu_path import dev, to_dev

pytestmark = pytest.mark.gpu

FLAGS = [0, 1, 3]  # plain, round_scale, round_scale + UE8M0
ROWS = 4  # MOE_FP8_SCALE_ROWS: receive-side scales row-major
LL_FLAGS = [0, 1, 3, 4, 5, 7]
Q_SENT = 0x57  # code byte pre-filled into receive rows
S_SENT = 0x7FC01234  # scale word pre-filled (a NaN: no real scale has it)


@pytest.fixture(scope="module")
def capi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_moe_layout_03_amd import capi as c

    return c


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _ref_scale_bits(qz, flags):
    return (qz["ue8m0"].view(np.uint32) if flags & 2 else qz["scale"].view(np.uint32))


def gpu_quantize(capi, xb: np.ndarray, flags: int):
    T, H = xb.shape
    cols = capi.fp8_scale_cols(H, flags)
    q = torch.full((T, H), Q_SENT, dtype=torch.uint8, device=dev())
    sd = torch.int32 if flags & 2 else torch.float32
    sc = torch.full((T, cols), 0, dtype=torch.int32, device=dev()).fill_(S_SENT) \
        .view(sd)
    capi.moe_quantize_fp8(T, H, to_dev(xb), q, sc, flags)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.view(torch.int32).cpu().numpy().view(np.uint32)


def check_quantize(capi, orc, xb, flags):
    q, sc = gpu_quantize(capi, xb, flags)
    ref = orc.quantize_fp8(xb, flags)
    bad = np.argwhere(q != ref["q"])
    assert bad.size == 0, ("codes", bad[:5], q[tuple(bad[0])], ref["q"][tuple(bad[0])])
    assert np.array_equal(sc, _ref_scale_bits(ref, flags)), "scales"


@pytest.mark.parametrize("flags", FLAGS)
def test_quantize_low_latency_batch(capi, orc, flags):
    w = mi.config_c3(128)
    _announce(f"quantize 128x7168 flags={flags}")
    check_quantize(capi, orc, w.x, flags)


def _crafted_rows():
    """Rows whose x / scale runs through every E4M3 value, every tie between
    adjacent values, and values one bf16 step either side of those ties, in
    both signs; the group maximum 3.5 makes the scale exactly 2^-7 (with and
    without round_scale), so x / scale = 128 x exactly and the hardware
    conversion alone decides each code."""
    import torch as _t

    vals = _t.arange(127, dtype=_t.int32).to(_t.uint8).view(_t.float8_e4m3fn).to(
        _t.float32).numpy().astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    targets = np.concatenate([vals, mids])
    xs = (targets / 128.0).astype(np.float32)
    xb = mi.to_bf16_bits(xs)
    assert np.array_equal(mi.bf16_bits_to_f32(xb).astype(np.float64) * 128.0, targets)
    up = xb + np.uint16(1)
    down = np.where(xb > 0, xb - np.uint16(1), xb).astype(np.uint16)
    pool = np.concatenate([xb, up, down, xb | np.uint16(0x8000), up | np.uint16(0x8000)])
    per = 127  # channel 0 of each group carries the 3.5
    groups = (pool.size + per - 1) // per
    H = 128 * int(np.ceil(groups / 4) * 4)
    row = np.zeros(H, np.uint16)
    three_half = mi.to_bf16_bits(np.array([3.5], np.float32))[0]
    for g in range(H // 128):
        row[g * 128] = three_half
        chunk = pool[g * per:(g + 1) * per]
        row[g * 128 + 1:g * 128 + 1 + chunk.size] = chunk
    return row[None, :]


@pytest.mark.parametrize("flags", FLAGS)
def test_quantize_crafted_ties_and_subnormals(capi, orc, flags):
    xb = _crafted_rows()
    _announce(f"quantize crafted E4M3 sweep H={xb.shape[1]} flags={flags}")
    check_quantize(capi, orc, xb, flags)


def _near_tie_rows():
    """Groups with non-power-of-two scales (every bf16 group maximum in [1, 2),
    and a few others) whose other channels are every bf16 x below the maximum
    for which x / scale lies within 4 float ulps of a midpoint between
    adjacent E4M3 values (about 1500 of them, both signs): the codes there
    depend on the quotient being the correctly rounded float, so they test the
    kernels' division and the conversion's tie handling together. Packed into
    rows of 2048 channels."""
    import torch as _t

    vals = _t.arange(127, dtype=_t.int32).to(_t.uint8).view(_t.float8_e4m3fn).to(
        _t.float32).numpy().astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    pats = (np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16).view(np.float32)  # positive normals
    amaxs = list((np.arange(0x3F80, 0x4000, dtype=np.uint32) << 16).view(np.float32))
    amaxs += [np.float32(v) for v in (0.01226806640625, 77.5, 0.005035400390625, 250.0)]
    groups = []
    for amax in amaxs:
        s = np.float32(amax) / np.float32(448.0)
        xs = pats[(pats > 0) & (pats < np.float32(amax))].astype(np.float64)
        q = xs / np.float64(s)
        j = np.clip(np.searchsorted(mids, q), 1, mids.size - 1)
        d = np.minimum(np.abs(q - mids[j]), np.abs(q - mids[j - 1]))
        ulp = np.spacing(q.astype(np.float32)).astype(np.float64)
        near = xs[d <= 4 * ulp].astype(np.float32)
        sel = np.concatenate([near, -near])
        for c in range(0, max(sel.size, 1), 127):
            g = np.zeros(128, np.float32)
            g[0] = amax
            part = sel[c:c + 127]
            g[1:1 + part.size] = part
            groups.append(g)
    while len(groups) % 16:
        groups.append(np.zeros(128, np.float32))
    return mi.to_bf16_bits(np.concatenate(groups).reshape(-1, 2048))


@pytest.mark.parametrize("flags", FLAGS)
def test_quantize_near_ties_with_inexact_scales(capi, orc, flags):
    xb = _near_tie_rows()
    _announce(f"quantize near-tie quotients H={xb.shape[1]} flags={flags}")
    check_quantize(capi, orc, xb, flags)


@pytest.mark.parametrize("flags", FLAGS)
def test_quantize_wide_range_and_zero_groups(capi, orc, flags):
    rng = np.random.default_rng(11)
    T, H = 37, 2048
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 20, (T, H // 128, 1))).astype(np.float32).repeat(
        128, axis=2).reshape(T, H)
    x[:, 128:256] = 0.0
    x[3] = 0.0
    x[:, 512:640] *= np.float32(1e-8)
    x[5, 700] = -0.0
    _announce(f"quantize wide range {T}x{H} flags={flags}")
    check_quantize(capi, orc, mi.to_bf16_bits(x), flags)


def run_ll_fp8(capi, w, M, src, flags, fused=True, rows=None):
    """moe_ll_layout_dispatch_fp8 (or moe_ll_layout + moe_ll_dispatch_fp8) into
    sentinel-filled buffers; returns (layout dict, recv_q, recv_scale words,
    status) with the receive tensors still on the GPU."""
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    lay = capi.LayoutBuffers.empty(shape, dev(), ll_M=M)
    for t in (lay.count, lay.offset, lay.slot, lay.rank_token_count, lay.row_src):
        t.fill_(-12345)
    lay.is_token_in_rank.fill_(7)
    full = w.E * w.R * M
    rows = full if rows is None else rows
    cols = capi.fp8_scale_cols(w.H, flags)
    rq = torch.full((full, w.H), Q_SENT, dtype=torch.uint8, device=dev())
    sshape = (full, cols) if flags & ROWS else (w.E, cols, w.R * M)
    rs = torch.empty(sshape, dtype=torch.int32, device=dev()).fill_(S_SENT)
    rs_arg = rs if flags & 2 else rs.view(torch.float32)
    idx = to_dev(w.topk_idx.astype(np.int64))
    nws = capi.moe_layout_workspace_bytes(shape)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev()) if nws else None
    x = to_dev(w.x)
    if fused:
        capi.moe_ll_layout_dispatch_fp8(shape, M, src, idx, lay, x, rq, rs_arg, rows, flags, ws)
    else:
        capi.moe_ll_layout(shape, M, src, idx, lay, ws)
        capi.moe_ll_dispatch_fp8(shape, M, x, lay.slot, rq, rs_arg, rows, flags, lay.status)
    torch.cuda.synchronize()
    got = dict(count=lay.count.cpu().numpy(), slot=lay.slot.cpu().numpy().reshape(w.T, w.K),
               status=int(lay.status.item()),
               rank_token_count=lay.rank_token_count.cpu().numpy(),
               is_token_in_rank=lay.is_token_in_rank.cpu().numpy().reshape(w.T, w.R),
               row_src=lay.row_src.cpu().numpy()[:w.E * M])
    return got, rq, rs, x


def check_ll_layout(got, ref):
    assert np.array_equal(got["slot"], ref["slot"]), "slot"
    assert np.array_equal(got["count"], ref["recv_count"]), "recv_count"
    assert np.array_equal(got["row_src"], ref["row_src"]), "row_src"
    assert np.array_equal(got["rank_token_count"], ref["rank_token_count"])
    assert np.array_equal(got["is_token_in_rank"], ref["is_token_in_rank"])
    assert got["status"] == ref["status"], (got["status"], ref["status"])


SMALL = [
    # (seed, T, H, E, R, K, M, src, neg, dup)
    (1, 13, 512, 16, 4, 3, 13, 2, 0.1, 0.2),
    (2, 8, 1024, 8, 2, 4, 9, 1, 0.0, 0.0),
    (3, 5, 640, 12, 4, 2, 7, 3, 0.3, 0.0),
    (4, 1, 128, 4, 4, 1, 1, 0, 0.0, 0.0),
    (5, 300, 512, 16, 4, 8, 300, 1, 0.05, 0.1),  # 2400 pairs: layout kernel + scatter
    (6, 64, 1536, 32, 8, 6, 64, 7, 0.0, 0.3),
]


@pytest.mark.parametrize("case", SMALL)
@pytest.mark.parametrize("flags", LL_FLAGS)
@pytest.mark.parametrize("fused", [True, False])
def test_ll_fp8_small_full(capi, orc, case, flags, fused):
    seed, T, H, E, R, K, M, src, neg, dup = case
    if flags & 2 and H % 512:
        pytest.skip("UE8M0 needs H % 512 == 0")
    w = mi.random_case(600 + seed, T, H, E, R, K, 1, neg_frac=neg, dup_frac=dup)
    _announce(f"ll fp8 small seed={seed} T={T} H={H} E={E} R={R} K={K} M={M} src={src} "
              f"flags={flags} fused={fused}")
    got, rq, rs, _ = run_ll_fp8(capi, w, M, src, flags, fused)
    ref = orc.ll_layout(w.topk_idx, E, R, M, src)
    check_ll_layout(got, ref)
    qz = orc.quantize_fp8(w.x, flags)
    fill_s = np.array([S_SENT], np.uint32).view(np.float32)[0]
    o = orc.ll_dispatch_fp8(qz, ref["slot"], E, R, M, flags, fill_q=Q_SENT, fill_scale=fill_s,
                            fill_ue=np.array([S_SENT], np.uint32).view(np.int32)[0])
    assert np.array_equal(rq.cpu().numpy(), o["recv_q"]), "codes"
    want = (o["recv_ue8m0"] if flags & 2 else o["recv_scale"]).view(np.uint32)
    assert np.array_equal(rs.cpu().numpy().view(np.uint32), want), "scales"


def _pairs(slot, T, K):
    v = slot.reshape(-1) >= 0
    rows = slot.reshape(-1)[v].astype(np.int64)
    toks = np.repeat(np.arange(T), K)[v]
    return rows, toks


def gpu_check_ll_fp8(rq, rs, qz, slot, w, M, flags):
    """Per pair, on the GPU: the row's codes and its scale column equal the
    oracle's cast of the token; every other row and scale entry keeps its
    sentinel."""
    rows, toks = _pairs(slot, w.T, w.K)
    rows_t = torch.from_numpy(rows).to(dev())
    toks_t = torch.from_numpy(toks).to(dev())
    q_ref = torch.from_numpy(qz["q"]).to(dev())
    s_ref = torch.from_numpy(np.ascontiguousarray(_ref_scale_bits(qz, flags)).view(np.int32)).to(
        dev())
    full = rq.shape[0]
    if flags & ROWS:
        rs_rows = rs  # already [rows, cols]
    else:
        cols = rs.shape[1]
        rs_rows = rs.permute(0, 2, 1).reshape(full, cols)  # [E, R*M, cols] -> rows
    for a in range(0, rows_t.numel(), 4096):
        r, t = rows_t[a:a + 4096], toks_t[a:a + 4096]
        assert torch.equal(rq[r], q_ref[t]), "codes"
        assert torch.equal(rs_rows[r], s_ref[t]), "scales"
    written = torch.zeros(full, dtype=torch.bool, device=dev())
    written[rows_t] = True
    step = 1 << 15
    for a in range(0, full, step):
        blk = rq[a:a + step][~written[a:a + step]]
        assert bool((blk == Q_SENT).all()), "untouched code rows"
    assert bool((rs_rows[~written] == S_SENT).all()), "untouched scales"


@pytest.mark.parametrize("M", mi.C3_SWEEP)
@pytest.mark.parametrize("flags", [0, 3, 4, 7])
def test_ll_fp8_sweep(capi, orc, M, flags):
    w = mi.config_c3(M)
    src = 5
    _announce(f"ll fp8 sweep M={M} src={src} flags={flags}")
    got, rq, rs, _ = run_ll_fp8(capi, w, M, src, flags)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, M, src)
    check_ll_layout(got, ref)
    gpu_check_ll_fp8(rq, rs, orc.quantize_fp8(w.x, flags), ref["slot"], w, M, flags)
    del rq, rs
    torch.cuda.empty_cache()


def test_ll_fp8_overflow(capi, orc):
    """An expert with more than M pairs (two picks of expert 2 per token, a
    duplicate id): the pairs past M get slot -1, are not written, and set the
    overflow bit."""
    w = mi.random_case(620, 40, 512, 16, 4, 4, 1)
    w.topk_idx[:, 0] = 2
    w.topk_idx[:, 1] = 2
    M = 40
    ref = orc.ll_layout(w.topk_idx, 16, 4, M, 1)
    assert ref["status"] & 2
    qz = orc.quantize_fp8(w.x, 3)
    for fused in (True, False):
        for flags in (3, 7):
            _announce(f"ll fp8 overflow M={M} fused={fused} flags={flags}")
            got, rq, rs, _ = run_ll_fp8(capi, w, M, 1, flags, fused)
            check_ll_layout(got, ref)
            gpu_check_ll_fp8(rq, rs, qz, ref["slot"], w, M, flags)


def test_ll_fp8_bad_slots(capi, orc):
    """moe_ll_dispatch_fp8 skips slots outside [-1, recv_rows) and flags them."""
    w = mi.random_case(621, 16, 512, 8, 2, 2, 1)
    M = 16
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, M, 0)
    slot = ref["slot"].copy()
    slot[3, 0] = -7
    slot[5, 1] = w.E * w.R * M + 3
    full = w.E * w.R * M
    rq = torch.full((full, w.H), Q_SENT, dtype=torch.uint8, device=dev())
    rs = torch.empty((w.E, 4, w.R * M), dtype=torch.int32, device=dev()).fill_(S_SENT)
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    _announce("ll fp8 bad slots")
    capi.moe_ll_dispatch_fp8(shape, M, to_dev(w.x), to_dev(slot.astype(np.int32)), rq,
                             rs.view(torch.float32), full, 0, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 4
    good = slot.copy()
    good[3, 0] = -1
    good[5, 1] = -1
    gpu_check_ll_fp8(rq, rs, orc.quantize_fp8(w.x, 0), good, w, M, 0)


@pytest.mark.parametrize("name", ["c1", "c2", "c4"])
def test_dispatch_fp8_tuple(capi, orc, name):
    """Buffer.dispatch with an (E4M3, scales) tuple, on the contiguous layout:
    both members bit for bit, untouched rows kept."""
    w = mi.by_name(name)
    H = w.H - w.H % 128
    qz = orc.quantize_fp8(np.ascontiguousarray(w.x[:, :H]), 0)
    A = 4 if name == "c1" else 1
    lay = orc.layout(w.topk_idx, w.E, w.R, A)
    rows = lay["rows"]
    shape = capi.make_shape(w.T, H, w.E, w.R, w.K, A)
    rq = torch.full((rows, H), Q_SENT, dtype=torch.uint8, device=dev())
    rs = torch.empty((rows, H // 128), dtype=torch.int32, device=dev()).fill_(0x7E577E57)
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    _announce(f"dispatch fp8 tuple {name} T={w.T} H={H}")
    capi.moe_dispatch_fp8(shape, to_dev(qz["q"]), to_dev(qz["scale"]),
                          to_dev(lay["slot"].astype(np.int32)), rq, rs.view(torch.float32), rows,
                          st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    want_q, want_s, _ = orc.dispatch_fp8_tuple(qz["q"], qz["scale"], lay["slot"], rows,
                                               fill16=0x5757)
    assert np.array_equal(rq.cpu().numpy(), want_q), "codes"
    got_s = rs.cpu().numpy().view(np.uint32)
    written = np.zeros(rows, bool)
    written[lay["slot"][lay["slot"] >= 0]] = True
    assert np.array_equal(got_s[written], want_s.view(np.uint32)[written]), "scales"
    assert np.all(got_s[~written] == 0x7E577E57), "untouched scales"


def test_fp8_empty_batch(capi):
    w = mi.random_case(622, 0, 512, 16, 4, 2, 1)
    _announce("ll fp8 T=0")
    got, rq, rs, _ = run_ll_fp8(capi, w, 8, 0, 3)
    assert got["count"].sum() == 0 and got["status"] == 0
    assert bool((rq == Q_SENT).all()) and bool((rs == S_SENT).all())
