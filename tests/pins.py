"""Pins of the oracle: checks against things other than the oracle itself.

Every check takes an ``Oracle`` (the normal build, or a build with a planted
mistake) and raises ``AssertionError`` when the oracle disagrees with

* the hand-worked example in ``golden/hand_worked_tiny.json``,
* the sort-based brute force in ``bruteforce.py``,
* numpy's library routines for the alignment-1 special case
  (``bincount`` / ``cumsum`` / stable ``argsort``),
* a dense matrix-product formulation of combine (``numpy`` matmul in f64),
* closed forms of combine with the identity expert (unit weights give K*x,
  softmax weights give x back after bf16 rounding, K=1 is a permutation
  round trip),
* the float error bound between the f32 and f64 combine sums,
* torch's CPU float->bf16 cast, and its float->float8_e4m3fn cast and
  float8 values,
* the hand-worked FP8 example in ``golden/fp8_hand_worked.json`` and the
  E4M3 rounding error bound of the per-128-channel cast,
* invariants (counts sum to the valid pairs; every pair has exactly one row;
  rows inside an expert increase with the pair index; offsets are multiples
  of the alignment; the replica tables are a bijection onto physical slots;
  replicated and unreplicated combine agree bit for bit).
"""
from __future__ import annotations

import json
import os

import numpy as np

import bruteforce as bf
import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_worked_tiny.json")


def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    g["idx"] = np.array(g["topk_idx"], np.int64)
    g["xb"] = mi.to_bf16_bits(np.array(g["x"], np.float32))
    g["w"] = np.array(g["topk_weights"], np.float32)
    return g


def check_golden(orc):
    g = _golden()
    ex = g["expected"]
    lay = orc.layout(g["idx"], g["E"], g["R"], g["A"])
    assert lay["count"].tolist() == ex["count"]
    assert lay["offset"].tolist() == ex["offset"]
    assert lay["slot"].tolist() == ex["slot"]
    assert lay["row_src"].tolist() == ex["row_src"]
    assert lay["is_token_in_rank"].tolist() == ex["is_token_in_rank"]
    assert lay["rank_token_count"].tolist() == ex["rank_token_count"]
    assert lay["status"] == 0
    recv, _ = orc.dispatch(g["xb"], lay["slot"], lay["rows"], fill=0)
    out = orc.combine(recv, lay["slot"], g["w"], "f64")["out_f64"]
    assert out.tolist() == ex["combine_identity"]
    rows = lay["rows"]
    y = mi.to_bf16_bits(np.array([[r + 1, (r + 1) / 2] for r in range(rows)], np.float32))
    for acc in ("f64", "f32"):
        res = orc.combine(y, lay["slot"], g["w"], acc)
        o = res["out_f64"] if acc == "f64" else res["out_f32"]
        assert o.tolist() == ex["combine_y_rows"], (acc, o.tolist())
        res1 = orc.combine(y, lay["slot"], None, acc)
        o1 = res1["out_f64"] if acc == "f64" else res1["out_f32"]
        assert o1.tolist() == ex["combine_y_rows_unit_weights"], (acc, o1.tolist())
    for key, M in (("ll_m4_s1", 4), ("ll_m3_s1", 3)):
        idx = np.array(ex[key].get("topk_idx", g["topk_idx"]), np.int64)
        ll = orc.ll_layout(idx, g["E"], g["R"], M, 1)
        assert ll["slot"].tolist() == ex[key]["slot"], (key, ll["slot"].tolist())
        assert ll["recv_count"].tolist() == ex[key]["recv_count"]
        assert ll["status"] == ex[key]["status"]
    rep = ex["replicas_c2"]
    plan = orc.plan_replicas(lay["count"], g["R"], 2)
    assert plan["replica_count"].tolist() == rep["replica_count"]
    assert plan["replica_phys"].tolist() == rep["replica_phys"]
    assert plan["phys_to_logical"].tolist() == rep["phys_to_logical"]
    phys, st = orc.reroute(g["idx"], g["E"], plan["replica_count"], plan["replica_phys"],
                           plan["E_phys"])
    assert phys.tolist() == rep["phys_idx"] and st == 0


def tiny_cases(n: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    for i in range(n):
        R = int(rng.choice([1, 2, 4]))
        E = R * int(rng.integers(1, 9))
        K = int(rng.integers(1, 9))
        T = int(rng.integers(0, 40))
        A = int(rng.choice([1, 2, 4, 16, 128]))
        yield mi.random_case(1000 * seed + i, T, 8, E, R, K, A,
                             neg_frac=float(rng.choice([0, 0.1, 0.5])),
                             dup_frac=float(rng.choice([0, 0.3])),
                             bad_frac=float(rng.choice([0, 0, 0.05])))


def check_layout_vs_bruteforce(orc, n: int = 150, seed: int = 0):
    for w in tiny_cases(n, seed):
        got = orc.layout(w.topk_idx, w.E, w.R, w.A)
        ref = bf.layout(w.topk_idx, w.E, w.R, w.A)
        tag = w.name
        assert got["count"].tolist() == ref["count"], tag
        assert got["offset"].tolist() == ref["offset"], tag
        assert got["slot"].tolist() == ref["slot"], tag
        assert got["row_src"].tolist() == ref["row_src"], tag
        assert got["is_token_in_rank"].tolist() == ref["is_token_in_rank"], tag
        assert got["rank_token_count"].tolist() == ref["rank_token_count"], tag
        assert bool(got["status"] & 1) == ref["bad"], tag


def check_ll_vs_bruteforce(orc, n: int = 100, seed: int = 1):
    rng = np.random.default_rng(seed)
    for w in tiny_cases(n, seed):
        if w.T == 0:
            continue
        M = int(w.T + rng.integers(0, 3))
        s = int(rng.integers(0, w.R))
        got = orc.ll_layout(w.topk_idx, w.E, w.R, M, s)
        ref = bf.ll_layout(w.topk_idx, w.E, w.R, M, s)
        assert got["slot"].tolist() == ref["slot"], w.name
        assert got["row_src"].tolist() == ref["row_src"], w.name
        assert got["recv_count"].tolist() == ref["recv_count"], w.name
        assert bool(got["status"] & 2) == ref["overflow"], w.name


def check_layout_vs_numpy(orc, workloads):
    """Alignment 1 reduces the layout to a counting sort of the flattened ids."""
    for w in workloads:
        ids = w.topk_idx.ravel()
        lay = orc.layout(w.topk_idx, w.E, w.R, 1)
        valid = ids >= 0
        cnt = np.bincount(ids[valid], minlength=w.E)
        assert np.array_equal(lay["count"], cnt), w.name
        assert np.array_equal(lay["offset"], np.concatenate([[0], np.cumsum(cnt)])), w.name
        order = np.argsort(np.where(valid, ids, w.E), kind="stable")[: int(valid.sum())]
        assert np.array_equal(lay["row_src"], order), w.name
        inv = np.full(ids.size, -1, np.int64)
        inv[order] = np.arange(order.size)
        assert np.array_equal(lay["slot"].ravel(), inv), w.name


def check_layout_invariants(orc, w, A: int = 1):
    lay = orc.layout(w.topk_idx, w.E, w.R, A)
    ids = w.topk_idx.ravel()
    slot = lay["slot"].ravel()
    valid = (ids >= 0) & (ids < w.E)
    assert lay["count"].sum() == valid.sum()
    assert np.all(lay["offset"] % A == 0)
    assert np.all(np.diff(lay["offset"]) >= lay["count"])
    assert np.all(np.diff(lay["offset"]) - lay["count"] < A)
    assert np.all(slot[~valid] == -1)
    vs = slot[valid]
    assert np.unique(vs).size == vs.size
    assert np.array_equal(lay["row_src"][vs], np.nonzero(valid)[0])
    e = ids[valid]
    lo = lay["offset"][e]
    assert np.all(vs >= lo) and np.all(vs < lo + lay["count"][e])
    # rows rise with the pair index inside each expert
    order = np.lexsort((np.nonzero(valid)[0], e))
    assert np.all(np.diff(vs[order])[np.diff(e[order]) == 0] == 1)
    in_rank = lay["is_token_in_rank"]
    assert np.array_equal(lay["rank_token_count"], in_rank.sum(axis=0))
    hit = np.zeros_like(in_rank)
    t_of = np.repeat(np.arange(w.T), w.K)[valid]
    hit[t_of, e // w.L] = 1
    assert np.array_equal(hit, in_rank)


def check_dispatch(orc, n: int = 40, seed: int = 2):
    for w in tiny_cases(n, seed):
        lay = orc.layout(w.topk_idx, w.E, w.R, w.A)
        rows = lay["rows"]
        recv, st = orc.dispatch(w.x, lay["slot"], rows, fill=0xABCD)
        assert st == 0
        for t in range(w.T):
            for k in range(w.K):
                s = lay["slot"][t, k]
                if s >= 0:
                    assert np.array_equal(recv[s], w.x[t]), w.name
        pad = lay["row_src"] < 0
        assert np.all(recv[pad] == 0xABCD), w.name


def check_combine_dense(orc, n: int = 40, seed: int = 3):
    for w in tiny_cases(n, seed):
        lay = orc.layout(w.topk_idx, w.E, w.R, w.A)
        rows = lay["rows"]
        rng = np.random.default_rng(w.seed)
        y = mi.to_bf16_bits(rng.standard_normal((rows, w.H), dtype=np.float32))
        yf = mi.bf16_bits_to_f32(y)
        for wt in (w.topk_weights, None):
            ref = bf.dense_combine(yf, lay["slot"], wt)
            got = orc.combine(y, lay["slot"], wt, "f64")["out_f64"]
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), w.name


def check_combine_closed_forms(orc, seed: int = 4):
    # K*x with unit weights (exact in f32 and f64), x with softmax weights
    for K in (1, 2, 6, 8):
        w = mi.random_case(seed + K, 64, 64, 32, 4, K, 1, distinct=True)
        lay = orc.layout(w.topk_idx, w.E, w.R, 1)
        recv, _ = orc.dispatch(w.x, lay["slot"], lay["rows"])
        xf = mi.bf16_bits_to_f32(w.x)
        o64 = orc.combine(recv, lay["slot"], None, "f64")["out_f64"]
        assert np.array_equal(o64, K * xf.astype(np.float64)), K
        r32 = orc.combine(recv, lay["slot"], None, "f32")
        assert np.array_equal(r32["out_f32"], (K * xf).astype(np.float32)), K
        soft = orc.combine(recv, lay["slot"], w.topk_weights, "f32")["out_bf16"]
        same = (soft == w.x) | ((xf == 0) & (mi.bf16_bits_to_f32(soft) == 0))
        assert np.all(same), K
        if K == 1:
            assert np.array_equal(orc.combine(recv, lay["slot"], None, "f32")["out_bf16"][xf != 0],
                                  w.x[xf != 0])
    # tokens whose ids are all -1 come back as +0
    w = mi.random_case(seed, 16, 16, 8, 2, 4, 1, neg_frac=1.0)
    lay = orc.layout(w.topk_idx, w.E, w.R, 1)
    r = orc.combine(np.zeros((1, 16), np.uint16), lay["slot"], w.topk_weights, "f32")
    assert np.all(r["out_bf16"] == 0)


def check_combine_f32_bound(orc, n: int = 30, seed: int = 5):
    """|f32 sum - f64 sum| <= K * 2^-24 * sum_k |w*y| (a K-term float sum)."""
    for w in tiny_cases(n, seed):
        lay = orc.layout(w.topk_idx, w.E, w.R, w.A)
        rng = np.random.default_rng(w.seed + 7)
        y = mi.to_bf16_bits(rng.standard_normal((max(lay["rows"], 1), w.H),
                                                dtype=np.float32) * 100)
        wt = (w.topk_weights * rng.uniform(-3, 3, w.topk_weights.shape)).astype(np.float32)
        o64 = orc.combine(y, lay["slot"], wt, "f64")["out_f64"]
        o32 = orc.combine(y, lay["slot"], wt, "f32")["out_f32"].astype(np.float64)
        yf = mi.bf16_bits_to_f32(y).astype(np.float64)
        mag = np.zeros_like(o64)
        for t in range(w.T):
            for k in range(w.K):
                s = lay["slot"][t, k]
                if s >= 0:
                    mag[t] += np.abs(wt[t, k] * yf[s])
        assert np.all(np.abs(o32 - o64) <= (w.K + 1) * 2.0 ** -24 * mag + 1e-30), w.name


def check_bf16_vs_torch(orc, n: int = 1 << 22, seed: int = 6):
    import torch

    rng = np.random.default_rng(seed)
    pats = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x807fffff, 0x3f808000, 0x3f818000,
                        0x3f80ffff, 0x3f817fff, 0x7f7fffff, 0x7f800000, 0xff800000, 0x7fc00000,
                        0xffc00001, 0x7f800001, 0x7f7f8000, 0x00008000, 0x00018000],
                       dtype=np.uint32)
    pats = np.concatenate([special, pats])
    f = pats.view(np.float32)
    got = orc.bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # the encoding of NaN is not fixed (torch's vector cast gives 0xFFFF, the
    # oracle the canonical 0x7FC0): NaN must stay NaN, everything else is bitwise
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(mi.bf16_bits_to_f32(got[nan])))


def check_replicas(orc, w, C_: int):
    lay = orc.layout(w.topk_idx, w.E, w.R, 1)
    load, st = orc.expert_load(w.topk_idx, w.E)
    assert np.array_equal(load, lay["count"]) and st == 0
    plan = orc.plan_replicas(load, w.R, C_)
    Ep, Lp = plan["E_phys"], plan["L_phys"]
    # hot set = the first C of a (load desc, id asc) library sort
    hot = np.lexsort((np.arange(w.E), -load.astype(np.int64)))[:C_]
    assert np.array_equal(np.sort(np.nonzero(plan["replica_count"] == 2)[0]), np.sort(hot))
    p2l = plan["phys_to_logical"]
    rp = plan["replica_phys"]
    # every physical slot maps back to its logical expert, and each physical
    # slot is used once
    used = np.concatenate([rp[:, 0], rp[rp[:, 1] >= 0, 1]])
    assert np.array_equal(np.sort(used), np.arange(Ep))
    assert np.all(p2l[rp[:, 0]] == np.arange(w.E))
    two = rp[:, 1] >= 0
    assert np.all(p2l[rp[two, 1]] == np.nonzero(two)[0])
    # primaries stay on the rank that owns the logical expert
    assert np.all(rp[:, 0] // Lp == np.arange(w.E) // w.L)
    phys, st = orc.reroute(w.topk_idx, w.E, plan["replica_count"], rp, Ep)
    assert st == 0
    v = w.topk_idx >= 0
    assert np.all(p2l[phys[v]] == w.topk_idx[v]) and np.all(phys[~v] == -1)
    # replica share = the odd tokens on hot experts
    plan_lay = orc.layout(phys, Ep, w.R, 1)
    t_of = np.repeat(np.arange(w.T), w.K).reshape(w.T, w.K)
    for i, e in enumerate(hot):
        odd = int(((w.topk_idx == e) & (t_of % 2 == 1)).sum())
        assert plan_lay["count"][rp[e, 1]] == odd
        assert plan_lay["count"][rp[e, 0]] + odd == load[e]
    # identity expert: replicated combine == unreplicated combine, bit for bit
    r0, _ = orc.dispatch(w.x, lay["slot"], lay["rows"])
    r1, _ = orc.dispatch(w.x, plan_lay["slot"], plan_lay["rows"])
    a = orc.combine(r0, lay["slot"], w.topk_weights, "f32")
    b = orc.combine(r1, plan_lay["slot"], w.topk_weights, "f32")
    assert np.array_equal(a["out_bf16"], b["out_bf16"])
    assert np.array_equal(a["out_f32"].view(np.uint32), b["out_f32"].view(np.uint32))


def check_ll_matches_contiguous(orc, w):
    """Source 0's padded layout and the contiguous layout give the same combine."""
    M = w.M or w.T
    ll = orc.ll_layout(w.topk_idx, w.E, w.R, M, 0)
    lay = orc.layout(w.topk_idx, w.E, w.R, 1)
    assert ll["status"] == 0
    assert np.array_equal(ll["recv_count"], lay["count"])
    r_ll, _ = orc.dispatch(w.x, ll["slot"], ll["rows"], fill=0)
    r_c, _ = orc.dispatch(w.x, lay["slot"], lay["rows"])
    a = orc.combine(r_ll, ll["slot"], w.topk_weights, "f32")["out_bf16"]
    b = orc.combine(r_c, lay["slot"], w.topk_weights, "f32")["out_bf16"]
    assert np.array_equal(a, b)
    # every used row decodes to (e, s=0, j) with j < recv_count[e]
    v = ll["slot"] >= 0
    rows = ll["slot"][v]
    e = rows // (w.R * M)
    s = (rows // M) % w.R
    j = rows % M
    assert np.array_equal(e, w.topk_idx[v]) and np.all(s == 0)
    assert np.all(j < ll["recv_count"][e])



# ---------------------------------------------------------------------------
# FP8 (E4M3 rows, one scale per 128 channels)
# ---------------------------------------------------------------------------
FP8_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                          "fp8_hand_worked.json")
ROUND, UE8M0, SCALE_ROWS = 1, 2, 4


def _fp8_golden_x(g):
    x = np.zeros((1, g["H"]), np.float32)
    for c, v in g["x"]:
        x[0, c] = v
    xb = mi.to_bf16_bits(x)
    # every listed value is exactly representable in bf16
    assert np.array_equal(mi.bf16_bits_to_f32(xb), x)
    return xb


def check_fp8_golden(orc):
    with open(FP8_GOLDEN) as f:
        g = json.load(f)
    xb = _fp8_golden_x(g)
    H = g["H"]
    for name, flags in (("plain", 0), ("round_scale", ROUND), ("round_scale", ROUND | UE8M0)):
        qz = orc.quantize_fp8(xb, flags)
        want = np.zeros(H, np.uint8)
        for c, code in g["codes"][name]:
            want[c] = code
        assert qz["q"][0].tolist() == want.tolist(), (name, np.nonzero(qz["q"][0] != want))
        sc = qz["scale"][0]
        if name == "plain":
            for gi, v in g["scale_exact"]["plain"].items():
                assert float(sc[int(gi)]) == v
            for gi, v in g["scale_approx"]["plain"].items():
                assert abs(float(sc[int(gi)]) - v) <= 1e-6 * v
        else:
            assert sc.tolist() == g["scale_exact"]["round_scale"]
        if flags & UE8M0:
            assert int(qz["ue8m0"][0, 0]) == g["ue8m0_word"]
    ll = g["ll"]
    idx = np.array(ll["topk_idx"], np.int64)
    lay = orc.ll_layout(idx, ll["E"], ll["R"], ll["M"], ll["src"])
    assert lay["slot"].tolist() == ll["slot"]
    qz = orc.quantize_fp8(xb, ROUND | UE8M0)
    out = orc.ll_dispatch_fp8(qz, lay["slot"], ll["E"], ll["R"], ll["M"], ROUND | UE8M0,
                              fill_q=0xAB, fill_scale=-1.0, fill_ue=-1)
    flat_s = out["recv_scale"].ravel()
    flat_u = out["recv_ue8m0"].ravel()
    touched_s, touched_u = set(), set()
    for row, sidx in ll["scale_index"].items():
        assert out["recv_q"][int(row)].tolist() == qz["q"][0].tolist()
        assert flat_s[sidx].tolist() == qz["scale"][0].tolist()
        assert int(flat_u[ll["ue8m0_index"][row]]) == g["ue8m0_word"]
        touched_s.update(sidx)
        touched_u.add(ll["ue8m0_index"][row])
    others = [i for i in range(flat_s.size) if i not in touched_s]
    assert np.all(flat_s[others] == -1.0)
    assert np.all(np.delete(flat_u, sorted(touched_u)) == -1)
    rows_used = {int(r) for r in ll["scale_index"]}
    for r in range(out["recv_q"].shape[0]):
        if r not in rows_used:
            assert np.all(out["recv_q"][r] == 0xAB)


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    import torch

    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values() -> np.ndarray:
    import torch

    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def check_e4m3_values_vs_torch(orc):
    """Code -> value for all 256 codes, against torch's float8_e4m3fn."""
    mine = orc.e4m3_value(np.arange(256, dtype=np.uint8))
    ref = _torch_e4m3_values()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def check_e4m3_vs_torch(orc, n: int = 1 << 20, seed: int = 7):
    """float -> E4M3 against torch's cast (round to nearest even) wherever the
    two readings agree (|v| <= 464: torch turns larger magnitudes into NaN,
    the reading here saturates them to 448, checked as a closed form)."""
    rng = np.random.default_rng(seed)
    vals = _torch_e4m3_values()
    fin = np.sort(np.unique(np.abs(vals[~np.isnan(vals)])))
    mids = (fin[:-1] + fin[1:]) / 2  # exact ties, as float32 (all representable)
    pats = np.arange(1 << 16, dtype=np.uint32) << 16
    allbf = pats.view(np.float32)
    allbf = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 464)]
    mags = np.exp2(rng.uniform(-14, 9, n)).astype(np.float32)
    sgn = np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    rnd = mags * sgn
    rnd = rnd[np.abs(rnd) <= 464]
    near = np.concatenate([mids, -mids]).astype(np.float32)
    near = np.concatenate([near, np.nextafter(near, np.float32(np.inf)),
                           np.nextafter(near, np.float32(-np.inf))])
    v = np.concatenate([allbf, rnd, near, np.array([0.0, -0.0, 448, -448, 464, -464],
                                                    np.float32)])
    v = v[np.abs(v) <= 464]
    got = orc.e4m3_from_f32(v)
    ref = _torch_e4m3(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])
    big = np.array([464.5, 480, 1e4, 3e38, -465, -1e30], np.float32)
    want = np.where(np.signbit(big), 0xFE, 0x7E).astype(np.uint8)
    assert orc.e4m3_from_f32(big).tolist() == want.tolist()


def _e4m3_half_ulp(a: np.ndarray) -> np.ndarray:
    """Half the E4M3 spacing at magnitude a (2^-10 in the subnormal range,
    2^(floor(log2 a) - 4) among normals)."""
    a = np.maximum(np.abs(a), 2.0 ** -6)
    return np.exp2(np.floor(np.log2(a)) - 4)


def check_quantize_properties(orc, xb: np.ndarray, flags: int):
    """Closed-form properties of the per-128-channel cast:
    * the scale is amax/448 to float rounding (round_scale: the smallest power
      of two >= that value), with amax floored at 1e-4;
    * without round_scale the group's largest magnitude gets the code for 448;
    * every code is within half an E4M3 spacing of x/scale (plus the float
      rounding of the division);
    * UE8M0 bytes are the scales' exponents, group 4w+b in byte b of word w."""
    qz = orc.quantize_fp8(xb, flags)
    T, H = xb.shape
    G = H // 128
    x = mi.bf16_bits_to_f32(xb).astype(np.float64).reshape(T, G, 128)
    s = qz["scale"].astype(np.float64)
    amax = np.maximum(np.abs(x).max(axis=2), np.float64(np.float32(1e-4)))
    ideal = amax / 448.0
    if flags & ROUND:
        m, e = np.frexp(s)
        assert np.all(m == 0.5), "round_scale scales must be powers of two"
        lo = ideal * (1 - 2.0 ** -23)
        assert np.all(s >= lo) and np.all(s / 2 < ideal * (1 + 2.0 ** -23))
    else:
        assert np.all(np.abs(s - ideal) <= ideal * 2.0 ** -24 * 1.0001)
    vals = orc.e4m3_value(np.arange(256, dtype=np.uint8))
    q = qz["q"].reshape(T, G, 128)
    dq = vals[q]
    assert not np.any(np.isnan(dq))
    r = x / s[:, :, None]
    tol = _e4m3_half_ulp(r) + np.abs(r) * 2.0 ** -23
    err = np.abs(dq - r)
    assert np.all(err <= tol), float((err - tol).max())
    # signs are kept, zeros included
    assert np.array_equal(np.signbit(dq), np.signbit(x))
    mag = np.abs(dq).max(axis=2)
    nonzero = np.abs(x).max(axis=2) >= np.float32(1e-4)
    if not (flags & ROUND):
        assert np.all(mag[nonzero] == 448.0)
    else:
        assert np.all((mag[nonzero] >= 224.0) & (mag[nonzero] <= 448.0))
    if flags & UE8M0:
        words = qz["ue8m0"].astype(np.int64) & 0xFFFFFFFF
        for b in range(4):
            byte = (words >> (8 * b)) & 0xFF
            assert np.array_equal(np.exp2(byte.astype(np.float64) - 127), s[:, b::4])


def check_fp8_cast_on_inputs(orc, n: int = 6, seed: int = 8):
    """check_quantize_properties on random bf16 rows with a wide dynamic range,
    all-zero groups and tiny groups."""
    rng = np.random.default_rng(seed)
    for i in range(n):
        T, H = int(rng.integers(1, 9)), 512 * int(rng.integers(1, 4))
        x = rng.standard_normal((T, H)).astype(np.float32)
        x *= np.exp2(rng.integers(-20, 12, (T, H // 128, 1))).astype(np.float32).repeat(
            128, axis=2).reshape(T, H)
        x[:, 128:256] = 0.0
        if H >= 512:
            x[:, 384:512] *= np.float32(1e-7)
        xb = mi.to_bf16_bits(x)
        for flags in (0, ROUND, ROUND | UE8M0):
            check_quantize_properties(orc, xb, flags)


def check_ll_fp8_dispatch(orc, n: int = 8, seed: int = 9):
    """Low-latency FP8 placement against numpy: every valid pair's row of codes
    is the token's codes, and reading the scale tensor as [E, R*M, G] (numpy
    transpose of the column-major storage) gives the token's scales on that
    row; everything else keeps its fill."""
    rng = np.random.default_rng(seed)
    for i in range(n):
        R = int(rng.choice([1, 2, 4]))
        E = R * int(rng.integers(1, 5))
        K = int(rng.integers(1, 5))
        M = int(rng.integers(1, 9))
        T = int(rng.integers(0, M + 1))
        w = mi.random_case(500 + i, T, 1024, E, R, K, neg_frac=0.2, dup_frac=0.2)
        src = int(rng.integers(0, R))
        lay = orc.ll_layout(w.topk_idx, E, R, M, src)
        for flags in (0, ROUND | UE8M0):
            qz = orc.quantize_fp8(w.x, flags)
            out = orc.ll_dispatch_fp8(qz, lay["slot"], E, R, M, flags, fill_q=0xCD,
                                      fill_scale=7.0, fill_ue=5)
            rows = E * R * M
            rs = out["recv_scale"].transpose(0, 2, 1).reshape(rows, 8)
            ru = out["recv_ue8m0"].transpose(0, 2, 1).reshape(rows, 2) if flags & UE8M0 \
                else None
            used = np.zeros(rows, bool)
            for t in range(T):
                for k in range(K):
                    r = lay["slot"][t, k]
                    if r < 0:
                        continue
                    used[r] = True
                    assert np.array_equal(out["recv_q"][r], qz["q"][t])
                    assert np.array_equal(rs[r], qz["scale"][t])
                    if ru is not None:
                        assert np.array_equal(ru[r], qz["ue8m0"][t])
            assert np.all(out["recv_q"][~used] == 0xCD)
            assert np.all(rs[~used] == 7.0)
            if ru is not None:
                assert np.all(ru[~used] == 5)
            # the row-major option: the scale tensors read directly as rows,
            # holding the same entries as the column-major ones
            rowm = orc.ll_dispatch_fp8(qz, lay["slot"], E, R, M, flags | SCALE_ROWS, fill_q=0xCD,
                                       fill_scale=7.0, fill_ue=5)
            assert np.array_equal(rowm["recv_q"], out["recv_q"])
            assert rowm["recv_scale"].shape == (rows, 8)
            assert np.array_equal(rowm["recv_scale"], rs)
            if ru is not None:
                assert np.array_equal(rowm["recv_ue8m0"], ru)


def check_combine_masked(orc, n: int = 30, seed: int = 10):
    """Masked combine against a dense formulation (numpy, f64): the weight of a
    pair on a masked rank is zeroed in W before W @ Y; the float sum is within
    the K-term float bound of it. Closed forms: no rank masked gives the plain
    combine bit for bit; every rank masked gives +0 everywhere."""
    rng = np.random.default_rng(seed)
    for i in range(n):
        R = int(rng.choice([1, 2, 4, 8]))
        E = R * int(rng.integers(1, 5))
        K = int(rng.integers(1, 7))
        T = int(rng.integers(1, 30))
        w = mi.random_case(800 + i, T, 16, E, R, K, neg_frac=0.2, dup_frac=0.2)
        lay = orc.layout(w.topk_idx, E, R, 1)
        y = mi.to_bf16_bits(rng.standard_normal((max(lay["rows"], 1), 16)).astype(np.float32))
        mask = (rng.random(R) < 0.4).astype(np.int32)
        got = orc.combine_masked(y, lay["slot"], w.topk_idx, E, R, mask, w.topk_weights)
        L = E // R
        W = np.zeros((T, y.shape[0]))
        absW = np.zeros((T, y.shape[0]))
        for t in range(T):
            for k in range(K):
                e, s_ = w.topk_idx[t, k], lay["slot"][t, k]
                if s_ < 0 or mask[e // L]:
                    continue
                W[t, s_] += w.topk_weights[t, k]
                absW[t, s_] += abs(float(w.topk_weights[t, k]))
        yf = mi.bf16_bits_to_f32(y).astype(np.float64)
        ref = W @ yf
        bound = (K + 1) * 2.0 ** -24 * (absW @ np.abs(yf)) + 1e-30
        assert np.all(np.abs(got["out_f32"].astype(np.float64) - ref) <= bound)
        none = orc.combine_masked(y, lay["slot"], w.topk_idx, E, R, np.zeros(R, np.int32),
                                  w.topk_weights)
        plain = orc.combine(y, lay["slot"], w.topk_weights, "f32")
        assert np.array_equal(none["out_f32"].view(np.uint32), plain["out_f32"].view(np.uint32))
        allm = orc.combine_masked(y, lay["slot"], w.topk_idx, E, R, np.ones(R, np.int32),
                                  w.topk_weights)
        assert np.all(allm["out_f32"].view(np.uint32) == 0)


def check_recv_stats(orc, seed: int = 11):
    """Cumulative receive counts: after n dispatches of the same batch the
    stats hold n times the per-expert receive counts (numpy bincount of the
    valid ids, capped at M for the low-latency layout)."""
    w = mi.random_case(900, 40, 16, 32, 4, 4, neg_frac=0.1, dup_frac=0.1)
    M = 40
    ll = orc.ll_layout(w.topk_idx, 32, 4, M, 1)
    ids = w.topk_idx[(w.topk_idx >= 0) & (w.topk_idx < 32)]
    want = np.minimum(np.bincount(ids, minlength=32), M)
    st = np.full(32, 5, np.int32)
    for n in range(1, 4):
        st = orc.accumulate_recv_stats(ll["recv_count"], st)
        assert np.array_equal(st, 5 + n * want)


def check_rank_golden(orc):
    g = _golden()
    ex = g["expected"]["ranks"]
    rl = orc.rank_layout(g["idx"], g["E"], g["R"], g["A"], g["w"])
    for key in ("rank_offset", "rank_slot", "recv_src", "recv_topk_idx", "recv_topk_weights",
                "recv_expert_count"):
        assert rl[key].tolist() == ex[key], (key, rl[key].tolist())
    recv, _ = orc.dispatch(g["xb"], rl["rank_slot"], rl["rows"], fill=0)
    out = orc.combine(recv, rl["rank_slot"], None, "f64")["out_f64"]
    assert out.tolist() == ex["combine_identity"]
    cw, st = orc.combine_rank_weights(rl["rank_slot"], rl["recv_topk_weights"])
    assert cw.tolist() == ex["combined_weights"] and st == 0


def check_rank_layout_vs_bruteforce(orc, n: int = 100, seed: int = 12):
    for w in tiny_cases(n, seed):
        got = orc.rank_layout(w.topk_idx, w.E, w.R, w.A, w.topk_weights)
        ref = bf.rank_layout(w.topk_idx, w.E, w.R, w.A, w.topk_weights)
        for key in ("rank_slot", "rank_offset", "recv_src", "recv_topk_idx",
                    "recv_expert_count"):
            assert np.array_equal(np.asarray(got[key]), np.asarray(ref[key])), key
        assert np.array_equal(got["recv_topk_weights"].view(np.uint32),
                              ref["recv_topk_weights"].view(np.uint32))


def check_rank_closed_forms(orc, w, A: int = 1):
    """Identity expert, no weights: a token's combined row is (ranks it
    reaches) x its row, exactly (small integer times a bf16 value); the
    weights summed back over ranks are the original ones (0 for -1 ids); the
    rank partitions hold the contiguous layout's distinct tokens per rank; the
    expert receive counts are numpy's bincount aligned to A."""
    rl = orc.rank_layout(w.topk_idx, w.E, w.R, A, w.topk_weights)
    lay = orc.layout(w.topk_idx, w.E, w.R, 1)
    assert np.array_equal(np.diff(rl["rank_offset"]), lay["rank_token_count"])
    ids = w.topk_idx[(w.topk_idx >= 0) & (w.topk_idx < w.E)]
    cnt = np.bincount(ids, minlength=w.E)
    assert np.array_equal(rl["recv_expert_count"], (cnt + A - 1) // A * A)
    recv, _ = orc.dispatch(w.x, rl["rank_slot"], max(rl["rows"], 1), fill=0)
    out = orc.combine(recv, rl["rank_slot"], None, "f32")["out_f32"]
    n = (rl["rank_slot"] >= 0).sum(axis=1).astype(np.float32)
    assert np.array_equal(out, n[:, None] * mi.bf16_bits_to_f32(w.x))
    cw, _ = orc.combine_rank_weights(rl["rank_slot"], rl["recv_topk_weights"])
    valid = (w.topk_idx >= 0) & (w.topk_idx < w.E)
    assert np.array_equal(cw, np.where(valid, w.topk_weights, 0.0).astype(np.float32))


def check_replica_sync_and_reduce(orc, seed: int = 13):
    """Weight sync and gradient reduction against numpy, through the other
    table of the plan (phys_to_logical): after the sync every physical slot
    holds its logical expert's master weights (numpy fancy indexing); the
    master gradient of expert e is numpy's float32 sum of the gradients of all
    physical slots that map to e (at most two terms: one rounding, so equal
    bit for bit); replicas of cold experts and all other slots are untouched."""
    rng = np.random.default_rng(seed)
    for E, R, C, S in ((16, 4, 4, 40), (64, 8, 16, 7), (8, 2, 0, 5), (32, 8, 32, 3)):
        load = rng.integers(0, 100, E).astype(np.int32)
        plan = orc.plan_replicas(load, R, C)
        Ep = plan["E_phys"]
        p2l = plan["phys_to_logical"]
        w = rng.integers(0, 1 << 16, (Ep, S)).astype(np.uint16)
        prim = plan["replica_phys"][:, 0]
        master = w[prim]  # the masters sit in the primary slots
        ws = orc.replica_weight_sync(w, plan["replica_count"], plan["replica_phys"])
        assert np.array_equal(ws, master[p2l])
        g = rng.standard_normal((Ep, S)).astype(np.float32)
        gr = orc.replica_grad_reduce(g, plan["replica_count"], plan["replica_phys"])
        want = np.zeros((E, S), np.float32)
        for e in range(E):
            terms = [g[p] for p in range(Ep) if p2l[p] == e]
            acc = terms[0]
            for tm in terms[1:]:
                acc = (acc + tm).astype(np.float32)
            want[e] = acc
        assert np.array_equal(gr[prim].view(np.uint32), want.view(np.uint32))
        others = np.ones(Ep, bool)
        others[prim] = False
        assert np.array_equal(gr[others].view(np.uint32), g[others].view(np.uint32))


ALL_SMALL_CHECKS = (
    check_golden,
    check_layout_vs_bruteforce,
    check_ll_vs_bruteforce,
    check_dispatch,
    check_combine_dense,
    check_combine_closed_forms,
    check_combine_f32_bound,
    check_fp8_golden,
    check_e4m3_values_vs_torch,
    lambda o: check_e4m3_vs_torch(o, n=1 << 14),
    lambda o: check_fp8_cast_on_inputs(o, n=2),
    lambda o: check_ll_fp8_dispatch(o, n=3),
    lambda o: check_combine_masked(o, n=8),
    check_recv_stats,
    check_rank_golden,
    lambda o: check_rank_layout_vs_bruteforce(o, n=30),
    check_replica_sync_and_reduce,
)
