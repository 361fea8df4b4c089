"""Parity of the HIP path (through the C ABI) with the oracle, element by element.

Bar: layout arrays, dispatched rows and untouched rows bit-exact; combine within
1e-2 relative + 1e-3 absolute of the oracle's f64 sum (the stated tolerance),
and, as a stronger check of the fixed summation order, bit-exact against the
oracle's f32 ascending-k sum and its bf16 rounding.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from gpu_path import SENTINEL, dev, np16, run_dispatch_combine, run_layout, to_dev

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-2, 1e-3


@pytest.fixture(scope="module")
def capi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_moe_layout_03_amd import capi as c

    return c


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check_layout(got, ref, w, ll=False):
    assert np.array_equal(got["slot"], ref["slot"]), "slot"
    if ll:
        assert np.array_equal(got["count"], ref["recv_count"]), "recv_count"
    else:
        assert np.array_equal(got["count"], ref["count"]), "count"
        assert np.array_equal(got["offset"], ref["offset"]), "offset"
    if "row_src" in got:
        assert np.array_equal(got["row_src"], ref["row_src"]), "row_src"
        assert np.array_equal(got["rank_token_count"], ref["rank_token_count"]), "rank_token_count"
        assert np.array_equal(got["is_token_in_rank"], ref["is_token_in_rank"]), "in_rank"
    assert got["status"] == ref["status"], ("status", got["status"], ref["status"])


def check_combine(orc, got16, got32, recv_ref, slot, wts, tokens=None):
    if tokens is not None:
        slot = slot[tokens]
        wts = None if wts is None else wts[tokens]
        got16 = got16[tokens]
        got32 = None if got32 is None else got32[tokens]
    r64 = orc.combine(recv_ref, slot, wts, "f64")["out_f64"]
    r32 = orc.combine(recv_ref, slot, wts, "f32")
    g16 = mi.bf16_bits_to_f32(got16).astype(np.float64)
    assert np.all(np.abs(g16 - r64) <= ATOL + RTOL * np.abs(r64)), "bf16 out vs f64 oracle"
    assert np.array_equal(got16, r32["out_bf16"]), "bf16 out vs f32-order oracle"
    if got32 is not None:
        g32 = got32.astype(np.float64)
        assert np.all(np.abs(g32 - r64) <= ATOL + RTOL * np.abs(r64)), "f32 out vs f64 oracle"
        assert np.array_equal(got32.view(np.uint32), r32["out_f32"].view(np.uint32)), \
            "f32 out vs f32-order oracle"


def full_case(capi, orc, w, A=None, weights=True):
    A = w.A if A is None else A
    got, lay, shape = run_layout(capi, w, A=A)
    ref = orc.layout(w.topk_idx, w.E, w.R, A)
    check_layout(got, ref, w)
    rows = ref["rows"]
    recv, o16, o32, st = run_dispatch_combine(capi, w, shape, lay, rows, weights=weights)
    rref, _ = orc.dispatch(w.x, ref["slot"], rows, fill=SENTINEL)
    assert np.array_equal(recv[:rows], rref), "dispatched rows / untouched padding"
    check_combine(orc, o16, o32, rref, ref["slot"], w.topk_weights if weights else None)
    assert st == ref["status"]


CASES = {
    "c1": lambda: mi.config_c1(),
    "c2": lambda: mi.config_c2(),
    "rand_ragged_H1000_K6": lambda: mi.random_case(11, 300, 1000, 64, 8, 6, 1, neg_frac=0.1),
    "rand_H8_K3_dups": lambda: mi.random_case(12, 77, 8, 12, 3, 3, 1, dup_frac=0.4),
    "rand_K1": lambda: mi.random_case(13, 200, 64, 16, 4, 1, 1),
    "rand_E1_R1": lambda: mi.random_case(14, 50, 16, 1, 1, 4, 1),
    "rand_E1024_R64": lambda: mi.random_case(15, 256, 128, 1024, 64, 8, 1),
    "rand_K64_onefull": lambda: mi.random_case(16, 128, 32, 256, 8, 64, 1),  # 8192 pairs
    "rand_K64_multi": lambda: mi.random_case(17, 129, 32, 256, 8, 64, 1),  # 8256 pairs
    # boundaries of the layout paths: one workgroup up to 1024 pairs (A > 1),
    # counting up to 4096 (A = 1), three launches above
    "rand_1024pairs": lambda: mi.random_case(23, 128, 64, 64, 8, 8, 1, neg_frac=0.02),
    "rand_1025pairs": lambda: mi.random_case(24, 1025, 16, 16, 4, 1, 1),
    "rand_4096pairs": lambda: mi.random_case(25, 512, 64, 256, 8, 8, 1),
    "rand_4097pairs": lambda: mi.random_case(26, 4097, 16, 32, 4, 1, 1),
    "rand_8193pairs": lambda: mi.random_case(18, 8193, 16, 32, 4, 1, 1),
    "rand_all_neg": lambda: mi.random_case(19, 64, 64, 16, 4, 4, 1, neg_frac=1.0),
    "rand_bad_ids": lambda: mi.random_case(20, 100, 64, 32, 4, 4, 1, bad_frac=0.1),
    "rand_T1": lambda: mi.random_case(21, 1, 7168, 256, 8, 8, 1, distinct=True),
    "rand_hot_expert": lambda: _hot(mi.random_case(22, 3000, 64, 64, 8, 6, 1), 5, 0.9),
    # the scatter: one workgroup per (token, 1 KiB chunk), two waves each
    # storing half the slots, four from 8192 chunks on when K >= 4. 8200
    # chunks with a ragged last chunk (125 vectors a row) and K = 3 (no
    # compile-time K, still two waves)
    "rand_wide_copy_ragged": lambda: mi.random_case(27, 4100, 1000, 64, 8, 3, 1, neg_frac=0.02),
    # four waves, no compile-time K: wave 0 takes slots 0 and 4
    "rand_split4_K5_ragged": lambda: mi.random_case(28, 4100, 1000, 64, 8, 5, 1, neg_frac=0.02),
    # four waves, K = 20: each wave's slots come in two groups of four
    "rand_split4_K20": lambda: mi.random_case(29, 2100, 2048, 64, 8, 20, 1),
    # either side of the 8192-chunk switch at K = 8 (two chunks a row)
    "rand_split2_K8_8190": lambda: mi.random_case(30, 4095, 1000, 256, 8, 8, 1),
    "rand_split4_K8_8192": lambda: mi.random_case(31, 4096, 1000, 256, 8, 8, 1),
    # K = 1: one wave per chunk, 16400 chunks
    "rand_split1_K1": lambda: mi.random_case(32, 8200, 1024, 32, 4, 1, 1),
}


def _hot(w, e, frac):
    """Send a fraction of all pairs to one expert (skew far beyond Zipf)."""
    rng = np.random.default_rng(w.seed)
    w.topk_idx = np.where(rng.random(w.topk_idx.shape) < frac, e, w.topk_idx)
    return w


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("A", [1, 16])
def test_path_parity(capi, orc, name, A):
    w = CASES[name]()
    _announce(f"{name} A={A} T={w.T} H={w.H} E={w.E} R={w.R} K={w.K}")
    full_case(capi, orc, w, A=A)


def test_max_row_width(capi, orc):
    """H = 2^20, the widest row the library takes, with 256 tokens: the
    scatter's and the combine's grids reach b * d = 2^32 (b: wave, d: waves
    per row), so a wave's token comes from a division there instead of the
    host reciprocal (exact only below that bound). Rows bit-exact, combine
    against the oracle on every token."""
    w = mi.random_case(28, 256, 1 << 20, 8, 2, 1, 1)
    _announce("max row width: T=256 H=2^20 E=8 R=2 K=1")
    got, lay, shape = run_layout(capi, w)
    ref = orc.layout(w.topk_idx, w.E, w.R, 1)
    check_layout(got, ref, w)
    rows = ref["rows"]
    recv, o16, _, st = run_dispatch_combine(capi, w, shape, lay, rows, f32=False)
    rref, _ = orc.dispatch(w.x, ref["slot"], rows, fill=SENTINEL)
    assert np.array_equal(recv[:rows], rref), "dispatched rows"
    del recv
    check_combine(orc, o16, None, rref, ref["slot"], w.topk_weights)
    assert st == ref["status"]


def test_unweighted_combine(capi, orc):
    w = mi.config_c2()
    _announce("c2 unweighted")
    full_case(capi, orc, w, weights=False)


def test_c2_alignment_128(capi, orc):
    w = mi.config_c2()
    _announce("c2 A=128")
    full_case(capi, orc, w, A=128)


def test_empty_batch(capi, orc):
    w = mi.random_case(30, 0, 64, 16, 4, 4, 4)
    _announce("T=0")
    got, lay, shape = run_layout(capi, w)
    assert got["count"].sum() == 0 and np.all(got["offset"] == 0)
    assert np.all(got["rank_token_count"] == 0) and got["status"] == 0
    recv, o16, o32, st = run_dispatch_combine(capi, w, shape, lay, 0)
    assert st == 0


def test_c4_skewed_full(capi, orc):
    w = mi.config_c4()
    _announce("c4 skewed full size")
    full_case(capi, orc, w)


def _gpu_rows_check(recv_t, x_t, slot, T, K):
    """On the GPU: every pair's row equals its token's row (bitwise); every
    other row still holds the sentinel."""
    v = slot.reshape(-1) >= 0
    rows_idx = torch.from_numpy(slot.reshape(-1)[v].astype(np.int64)).to(dev())
    toks = torch.from_numpy(np.repeat(np.arange(T), K)[v]).to(dev())
    for a in range(0, rows_idx.numel(), 4096):
        assert torch.equal(recv_t[rows_idx[a:a + 4096]], x_t[toks[a:a + 4096]])
    written = torch.zeros(recv_t.shape[0], dtype=torch.bool, device=dev())
    written[rows_idx] = True
    sent = SENTINEL - 65536 if SENTINEL > 32767 else SENTINEL
    step = 1 << 16
    for a in range(0, recv_t.shape[0], step):
        blk = recv_t[a:a + step][~written[a:a + step]]
        assert bool((blk == sent).all())


def test_c5_replica_path_full(capi, orc):
    """Replica workload at full size: reroute + layout + dispatch + combine;
    the combine of all 8192 tokens matches the oracle, and equals the
    unreplicated path bit for bit."""
    w = mi.config_c5()
    _announce("c5 replica full size")
    C_ = w.replicas
    d_idx = to_dev(w.topk_idx)
    load = torch.empty(w.E, dtype=torch.int32, device=dev())
    status = torch.zeros(1, dtype=torch.int32, device=dev())
    capi.moe_expert_load(w.T, w.K, w.E, d_idx, load, status)
    rc = torch.full((w.E,), -7, dtype=torch.int32, device=dev())
    rp = torch.full((w.E, 2), -7, dtype=torch.int32, device=dev())
    p2l = torch.full((w.E + C_,), -7, dtype=torch.int32, device=dev())
    capi.moe_plan_replicas(w.E, w.R, C_, load, rc, rp, p2l)
    phys = torch.full((w.T, w.K), -7, dtype=torch.int64, device=dev())
    capi.moe_reroute(w.T, w.K, w.E, d_idx, rc, rp, w.E + C_, phys, status)
    torch.cuda.synchronize()
    load_ref, _ = orc.expert_load(w.topk_idx, w.E)
    assert np.array_equal(load.cpu().numpy(), load_ref)
    plan = orc.plan_replicas(load_ref, w.R, C_)
    assert np.array_equal(rc.cpu().numpy(), plan["replica_count"])
    assert np.array_equal(rp.cpu().numpy(), plan["replica_phys"])
    assert np.array_equal(p2l.cpu().numpy(), plan["phys_to_logical"])
    phys_ref, st = orc.reroute(w.topk_idx, w.E, plan["replica_count"], plan["replica_phys"],
                               plan["E_phys"])
    assert np.array_equal(phys.cpu().numpy(), phys_ref) and int(status.item()) == 0 == st

    Ep = plan["E_phys"]
    got, lay, shape = run_layout(capi, w, idx=phys_ref, E=Ep)
    ref = orc.layout(phys_ref, Ep, w.R, 1)
    check_layout(got, ref, w)
    rows = ref["rows"]
    recv_t = torch.full((rows, w.H), SENTINEL, dtype=torch.int16, device=dev())
    x_t = to_dev(w.x)
    capi.moe_dispatch(shape, x_t, lay.slot, recv_t, rows, lay.status)
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev())
    o32 = torch.empty(w.T, w.H, dtype=torch.float32, device=dev())
    wt = to_dev(w.topk_weights)
    capi.moe_combine(shape, recv_t, rows, lay.slot, wt, out, o32, lay.status)
    torch.cuda.synchronize()
    _gpu_rows_check(recv_t, x_t, ref["slot"], w.T, w.K)
    # every token against the oracle's own dispatch of the physical layout:
    # bf16 and f32 bit-exact against its f32 ascending-k sum, and within the
    # 1e-2 / 1e-3 tolerance of its f64 sum
    rref, _ = orc.dispatch(w.x, ref["slot"], rows)
    check_combine(orc, np16(out), o32.cpu().numpy(), rref, ref["slot"], w.topk_weights)
    del rref
    # the unreplicated path gives the same bits
    sh2 = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    lay2 = capi.LayoutBuffers.empty(sh2, dev())
    ws = torch.empty(capi.moe_layout_workspace_bytes(sh2), dtype=torch.uint8, device=dev())
    capi.moe_layout(sh2, d_idx, lay2, ws)
    rows2 = w.T * w.K
    recv2 = torch.empty(rows2, w.H, dtype=torch.int16, device=dev())
    capi.moe_dispatch(sh2, x_t, lay2.slot, recv2, rows2, lay2.status)
    out2 = torch.empty_like(out)
    o32b = torch.empty_like(o32)
    capi.moe_combine(sh2, recv2, rows2, lay2.slot, wt, out2, o32b, lay2.status)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(o32.view(torch.int32), o32b.view(torch.int32))
    assert int(lay.status.item()) == 0 and int(lay2.status.item()) == 0


@pytest.mark.parametrize("M", mi.C3_SWEEP)
def test_ll_sweep(capi, orc, M):
    w = mi.config_c3(M)
    s = 0 if M != 128 else 7
    _announce(f"c3 LL M={M} src={s}")
    got, lay, shape = run_layout(capi, w, ll=True, M=M, src=s)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, M, s)
    check_layout(got, ref, w, ll=True)
    rows = ref["rows"]
    x_t = to_dev(w.x)
    recv_t = torch.full((rows, w.H), SENTINEL, dtype=torch.int16, device=dev())
    capi.moe_dispatch(shape, x_t, lay.slot, recv_t, rows, lay.status)
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev())
    o32 = torch.empty(w.T, w.H, dtype=torch.float32, device=dev())
    capi.moe_combine(shape, recv_t, rows, lay.slot, to_dev(w.topk_weights), out, o32, lay.status)
    torch.cuda.synchronize()
    _gpu_rows_check(recv_t, x_t, ref["slot"], w.T, w.K)
    # combine: the oracle reads its own padded rows; compact them to the used rows
    v = ref["slot"] >= 0
    used = np.unique(ref["slot"][v])
    remap = np.full(rows, -1, np.int64)
    remap[used] = np.arange(used.size)
    slot_c = np.where(v, remap[np.maximum(ref["slot"], 0)], -1).astype(np.int32)
    rref, _ = orc.dispatch(w.x, slot_c, used.size)
    check_combine(orc, np16(out), o32.cpu().numpy(), rref, slot_c, w.topk_weights)
    assert int(lay.status.item()) == 0
    del recv_t
    torch.cuda.empty_cache()


def test_ll_overflow_and_small_M(capi, orc):
    w = _hot(mi.random_case(40, 30, 64, 16, 4, 4, 1), 5, 0.9)
    _announce("LL overflow on a hot expert, M=30")
    got, lay, shape = run_layout(capi, w, ll=True, M=30, src=2)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, 30, 2)
    assert ref["status"] & 2
    check_layout(got, ref, w, ll=True)


def test_ll_multiblock(capi, orc):
    w = mi.random_case(41, 2000, 64, 64, 8, 6, 1, M=2000, neg_frac=0.05)  # 12000 pairs
    _announce("LL multi-block M=2000")
    got, lay, shape = run_layout(capi, w, ll=True, M=2000, src=5)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, 2000, 5)
    check_layout(got, ref, w, ll=True)


def test_ll_multiblock_overflow(capi, orc):
    w = _hot(mi.random_case(42, 1500, 16, 8, 2, 8, 1, M=1500), 3, 0.5)
    _announce("LL multi-block overflow")
    got, lay, shape = run_layout(capi, w, ll=True, M=1500, src=1)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, 1500, 1)
    assert ref["status"] & 2
    check_layout(got, ref, w, ll=True)


def test_bad_slots_are_skipped(capi, orc):
    w = mi.random_case(43, 64, 64, 16, 4, 4, 1)
    _announce("bad slots")
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    ref = orc.layout(w.topk_idx, w.E, w.R, 1)
    slot = ref["slot"].copy()
    slot[3, 1] = 10_000_000
    slot[5, 0] = -5
    rows = ref["rows"]
    x_t = to_dev(w.x)
    recv_t = torch.full((rows, w.H), SENTINEL, dtype=torch.int16, device=dev())
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    capi.moe_dispatch(shape, x_t, to_dev(slot), recv_t, rows, st)
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev())
    st2 = torch.zeros(1, dtype=torch.int32, device=dev())
    capi.moe_combine(shape, recv_t, rows, to_dev(slot), to_dev(w.topk_weights), out, None, st2)
    torch.cuda.synchronize()
    rref, rst = orc.dispatch(w.x, slot, rows, fill=SENTINEL)
    assert np.array_equal(np16(recv_t), rref) and int(st.item()) == rst == 4
    cref = orc.combine(rref, slot, w.topk_weights, "f32")
    assert np.array_equal(np16(out), cref["out_bf16"]) and int(st2.item()) == 4


def test_replica_small_and_ties(capi, orc):
    for seed, (T, E, R, K, C_) in enumerate([(50, 16, 4, 3, 4), (64, 8, 8, 2, 8), (10, 64, 8, 8, 0),
                                             (300, 256, 8, 8, 32), (5, 1024, 8, 4, 64)]):
        w = mi.random_case(50 + seed, T, 16, E, R, K, 1, neg_frac=0.1)
        _announce(f"replica plan T={T} E={E} R={R} C={C_}")
        d_idx = to_dev(w.topk_idx)
        load = torch.empty(E, dtype=torch.int32, device=dev())
        capi.moe_expert_load(T, K, E, d_idx, load)
        rc = torch.empty(E, dtype=torch.int32, device=dev())
        rp = torch.empty(E, 2, dtype=torch.int32, device=dev())
        p2l = torch.empty(E + C_, dtype=torch.int32, device=dev())
        capi.moe_plan_replicas(E, R, C_, load, rc, rp, p2l)
        phys = torch.empty(T, K, dtype=torch.int64, device=dev())
        capi.moe_reroute(T, K, E, d_idx, rc, rp, E + C_, phys)
        torch.cuda.synchronize()
        lref, _ = orc.expert_load(w.topk_idx, E)
        plan = orc.plan_replicas(lref, R, C_)
        pref, _ = orc.reroute(w.topk_idx, E, plan["replica_count"], plan["replica_phys"],
                              plan["E_phys"])
        assert np.array_equal(load.cpu().numpy(), lref)
        assert np.array_equal(rc.cpu().numpy(), plan["replica_count"])
        assert np.array_equal(rp.cpu().numpy(), plan["replica_phys"])
        assert np.array_equal(p2l.cpu().numpy(), plan["phys_to_logical"])
        assert np.array_equal(phys.cpu().numpy(), pref)


def test_expert_load_bad_ids(capi, orc):
    w = mi.random_case(60, 5000, 8, 64, 8, 6, 1, bad_frac=0.02, neg_frac=0.1)
    _announce("expert load with bad ids, 30000 pairs")
    load = torch.empty(w.E, dtype=torch.int32, device=dev())
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    capi.moe_expert_load(w.T, w.K, w.E, to_dev(w.topk_idx), load, st)
    torch.cuda.synchronize()
    lref, sref = orc.expert_load(w.topk_idx, w.E)
    assert np.array_equal(load.cpu().numpy(), lref) and int(st.item()) == sref == 1


def test_deterministic_runs(capi, orc):
    """Two runs of the skewed workload give identical bytes (no order depends
    on atomics)."""
    w = mi.config_c4()
    _announce("c4 determinism")
    outs = []
    for _ in range(2):
        got, lay, shape = run_layout(capi, w)
        recv, o16, o32, st = run_dispatch_combine(capi, w, shape, lay, got["rows"])
        outs.append((got["slot"].copy(), recv.copy(), o16.copy(), o32.copy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


# -- layout and dispatch in one call -------------------------------------------

from gpu_path import run_layout_dispatch  # noqa: E402

FUSED_CASES = {k: v for k, v in CASES.items()
               if k not in ("rand_8193pairs", "rand_K64_onefull", "rand_K64_multi")}
FUSED_CASES["rand_2048pairs"] = lambda: mi.random_case(70, 256, 520, 96, 8, 8, 1, neg_frac=0.05)
FUSED_CASES["rand_2049pairs"] = lambda: mi.random_case(71, 2049, 64, 32, 4, 1, 1)
# wide rows: 300 tokens of 14 row chunks with a ragged 2400-pair routing,
# 256 tokens of 20 chunks; from 512 tokens on each copying wave takes two
# chunks and a row needs one workgroup (14 chunks), or two of 10 (20 chunks)
FUSED_CASES["rand_T300_wide"] = lambda: mi.random_case(75, 300, 7168, 256, 8, 8, 1, neg_frac=0.02,
                                                       dup_frac=0.02)
FUSED_CASES["rand_T256_H10240"] = lambda: mi.random_case(76, 256, 10240, 256, 8, 8, 1)
FUSED_CASES["rand_T512_wide"] = lambda: mi.random_case(78, 512, 7168, 256, 8, 8, 1, neg_frac=0.01,
                                                       dup_frac=0.02)
FUSED_CASES["rand_T512_H10240"] = lambda: mi.random_case(79, 512, 10240, 64, 8, 8, 1,
                                                         neg_frac=0.02)
FUSED_CASES["rand_T600_H1000"] = lambda: mi.random_case(80, 600, 1000, 64, 8, 6, 1, neg_frac=0.02)
# the counting kernel's largest keys: 1024 experts x 4096 pairs
FUSED_CASES["rand_E1024_4096pairs"] = lambda: mi.random_case(72, 512, 64, 1024, 64, 8, 1,
                                                             neg_frac=0.02, dup_frac=0.05,
                                                             bad_frac=0.01)


@pytest.mark.parametrize("name", sorted(FUSED_CASES))
@pytest.mark.parametrize("A", [1, 16])
def test_layout_dispatch_parity(capi, orc, name, A):
    w = FUSED_CASES[name]()
    _announce(f"layout_dispatch {name} A={A} T={w.T} H={w.H} E={w.E} R={w.R} K={w.K}")
    got, recv_t, lay, shape = run_layout_dispatch(capi, w, A=A)
    ref = orc.layout(w.topk_idx, w.E, w.R, A)
    check_layout(got, ref, w)
    rows = ref["rows"]
    rref, _ = orc.dispatch(w.x, ref["slot"], rows, fill=SENTINEL)
    recv = np16(recv_t)
    assert np.array_equal(recv[:rows], rref), "dispatched rows / untouched padding"
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev())
    o32 = torch.empty(w.T, w.H, dtype=torch.float32, device=dev())
    capi.moe_combine(shape, recv_t, recv_t.shape[0], lay.slot, to_dev(w.topk_weights), out, o32,
                     lay.status)
    torch.cuda.synchronize()
    check_combine(orc, np16(out), o32.cpu().numpy(), rref, ref["slot"], w.topk_weights)


@pytest.mark.parametrize("M", mi.C3_SWEEP)
def test_ll_layout_dispatch_sweep(capi, orc, M):
    w = mi.config_c3(M)
    s = 3
    _announce(f"ll_layout_dispatch M={M} src={s}")
    got, recv_t, lay, shape = run_layout_dispatch(capi, w, ll=True, M=M, src=s)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, M, s)
    check_layout(got, ref, w, ll=True)
    _gpu_rows_check(recv_t, to_dev(w.x), ref["slot"], w.T, w.K)
    del recv_t
    torch.cuda.empty_cache()


def test_layout_dispatch_empty_and_overflow(capi, orc):
    w = mi.random_case(72, 0, 64, 16, 4, 4, 2)
    _announce("layout_dispatch T=0")
    got, recv_t, lay, shape = run_layout_dispatch(capi, w)
    assert got["count"].sum() == 0 and np.all(got["offset"] == 0) and got["status"] == 0
    assert np.all(got["rank_token_count"] == 0)
    w = _hot(mi.random_case(73, 40, 64, 16, 4, 4, 1), 2, 0.9)
    _announce("ll_layout_dispatch overflow M=40")
    got, recv_t, lay, shape = run_layout_dispatch(capi, w, ll=True, M=40, src=1)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, 40, 1)
    assert ref["status"] & 2
    check_layout(got, ref, w, ll=True)
    _gpu_rows_check(recv_t, to_dev(w.x), ref["slot"], w.T, w.K)


@pytest.mark.parametrize("M", [256, 120])
def test_ll_layout_dispatch_hot_stripe(capi, orc, M):
    """A stripe with more pairs than a duty workgroup stages in LDS (64): its
    later rows are stored one by one; at M = 120 the stripe also overflows."""
    w = _hot(mi.random_case(77, 120, 64, 32, 4, 8, 1, neg_frac=0.03, dup_frac=0.05), 5, 0.2)
    _announce(f"ll_layout_dispatch hot stripe M={M}")
    got, recv_t, lay, shape = run_layout_dispatch(capi, w, ll=True, M=M, src=2)
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, M, 2)
    assert int(np.max(np.bincount(w.topk_idx[w.topk_idx >= 0], minlength=w.E))) > 64
    check_layout(got, ref, w, ll=True)
    _gpu_rows_check(recv_t, to_dev(w.x), ref["slot"], w.T, w.K)


@pytest.mark.parametrize("T", [1, 2, 40])
def test_ll_few_tokens_many_stripes(capi, orc, T):
    """More stripes than the copying workgroups empty (8 each): the rest are
    the duty workgroups', in the layout-only and the fused launch."""
    w = mi.random_case(78 + T, T, 2048, 256, 8, 8, 1, neg_frac=0.05)
    M = T + 3
    ref = orc.ll_layout(w.topk_idx, w.E, w.R, M, 6)
    _announce(f"ll_layout T={T} E=256 M={M}")
    got, lay, shape = run_layout(capi, w, ll=True, M=M, src=6)
    check_layout(got, ref, w, ll=True)
    _announce(f"ll_layout_dispatch T={T} E=256 M={M}")
    got, recv_t, lay, shape = run_layout_dispatch(capi, w, ll=True, M=M, src=6)
    check_layout(got, ref, w, ll=True)
    _gpu_rows_check(recv_t, to_dev(w.x), ref["slot"], w.T, w.K)


def test_layout_dispatch_small_receive_buffer(capi, orc):
    """Rows at or past recv_rows are skipped and flagged, never written."""
    w = mi.random_case(74, 64, 64, 16, 4, 4, 1)
    _announce("layout_dispatch with recv_rows = 100 < 256")
    got, recv_t, lay, shape = run_layout_dispatch(capi, w, rows=100)
    ref = orc.layout(w.topk_idx, w.E, w.R, 1)
    assert np.array_equal(got["slot"], ref["slot"])
    rref, st = orc.dispatch(w.x, ref["slot"], 100, fill=SENTINEL)
    assert st == 4 and got["status"] == 4
    assert np.array_equal(np16(recv_t), rref)


def test_graph_replays_match_eager(capi, orc):
    """The standard step captured in a HIP graph: every replay, with eager
    work and synchronisation between replays, reproduces the eager outputs
    (layout arrays, receive rows, combine) bit for bit."""
    w = mi.config_c2()
    _announce("graph capture of layout_dispatch + combine, 4 replays")
    shape = capi.make_shape(w.T, w.H, w.E, w.R, w.K, 1)
    idx, x, wt = to_dev(w.topk_idx), to_dev(w.x), to_dev(w.topk_weights)
    lay = capi.LayoutBuffers.empty(shape, dev())
    rows = capi.moe_recv_rows_worst(shape)
    recv = torch.zeros(rows, w.H, dtype=torch.int16, device=dev())
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev())
    stream = torch.cuda.Stream()

    def step():
        capi.moe_layout_dispatch(shape, idx, lay, x, recv, rows, stream=stream)
        capi.moe_combine(shape, recv, rows, lay.slot, wt, out, None, lay.status, stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (lay.count, lay.offset, lay.slot, lay.row_src, lay.rank_token_count,
                               lay.is_token_in_rank, recv, out)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for rep in range(4):
        for t in (lay.count, lay.offset, lay.slot, out):
            t.fill_(-3)
        recv.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (lay.count, lay.offset, lay.slot, lay.row_src, lay.rank_token_count,
               lay.is_token_in_rank, recv, out)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        junk = torch.randn(1 << 20, device=dev()).sum()  # eager work between replays
        assert torch.isfinite(junk)
    ref_lay = orc.layout(w.topk_idx, w.E, w.R, 1)
    assert np.array_equal(lay.slot.cpu().numpy().reshape(w.T, w.K), ref_lay["slot"])
    assert int(lay.status.item()) == 0


def test_special_values_bit_patterns(capi, orc):
    """Rows of arbitrary bf16 bit patterns (NaN, infinities, -0, subnormals
    included) and weights of any sign and size: dispatch copies the bits,
    combine matches the oracle's float ascending-k path bit for bit (NaN
    results as 0x7FC0; subnormal products kept, not flushed)."""
    rng = np.random.default_rng(99)
    w = mi.random_case(99, 200, 264, 32, 4, 6, 1, neg_frac=0.1, dup_frac=0.2)
    x = rng.integers(0, 1 << 16, (w.T, w.H)).astype(np.uint16)
    x[:, :8] = np.array([0x7F80, 0xFF80, 0x7FC1, 0x8000, 0x0001, 0x807F, 0x0080, 0x7F7F],
                        np.uint16)
    wts = (rng.standard_normal((w.T, w.K)) * np.exp2(rng.integers(-130, 20, (w.T, w.K)))
           ).astype(np.float32)
    wts[0, :] = 0.0
    wts[1, 0] = -0.0
    w.topk_weights = wts
    _announce("special bit patterns: dispatch + weighted combine")
    got, lay, shape = run_layout(capi, w)
    ref = orc.layout(w.topk_idx, w.E, w.R, 1)
    check_layout(got, ref, w)
    recv, out16, out32, st = run_dispatch_combine(capi, w, shape, lay, got["rows"], x=x)
    rref, _ = orc.dispatch(x, ref["slot"], got["rows"], fill=SENTINEL)
    assert np.array_equal(recv[:got["rows"]], rref), "dispatch bits"
    r32 = orc.combine(rref, ref["slot"], wts, "f32")
    assert np.array_equal(out16, r32["out_bf16"]), "combine bf16 bits"
    g, r = out32.view(np.uint32), r32["out_f32"].view(np.uint32)
    nan = np.isnan(r32["out_f32"])
    assert np.array_equal(np.isnan(out32), nan)
    assert np.array_equal(g[~nan], r[~nan]), "combine f32 bits"
