"""The oracle against its pins (CPU only). See pins.py for what each pin is."""
import numpy as np
import pytest

import moe_inputs as mi
import pins


def test_golden_hand_worked(orc):
    pins.check_golden(orc)


def test_layout_vs_bruteforce(orc):
    pins.check_layout_vs_bruteforce(orc, n=300, seed=0)


def test_ll_layout_vs_bruteforce(orc):
    pins.check_ll_vs_bruteforce(orc, n=200, seed=1)


def test_dispatch_rows_and_untouched_padding(orc):
    pins.check_dispatch(orc, n=60)


def test_combine_vs_dense_matmul(orc):
    pins.check_combine_dense(orc, n=60)


def test_combine_closed_forms(orc):
    pins.check_combine_closed_forms(orc)


def test_combine_f32_within_float_bound_of_f64(orc):
    pins.check_combine_f32_bound(orc, n=60)


def test_bf16_rounding_matches_torch_cpu(orc):
    pins.check_bf16_vs_torch(orc)


@pytest.mark.parametrize("name", ["c1", "c2", "c3_m16", "c3_m512", "c4", "c5"])
def test_layout_vs_numpy_library_at_config(orc, name):
    pins.check_layout_vs_numpy(orc, [mi.by_name(name)])


@pytest.mark.parametrize("name,A", [("c1", 1), ("c1", 16), ("c2", 1), ("c2", 128), ("c4", 4),
                                    ("c5", 1), ("c5", 64)])
def test_layout_invariants_at_config(orc, name, A):
    pins.check_layout_invariants(orc, mi.by_name(name), A)


@pytest.mark.parametrize("M", mi.C3_SWEEP)
def test_ll_equals_contiguous_for_source_zero(orc, M):
    w = mi.config_c3(M)
    if M >= 256:  # keep the CPU suite quick: the property is per token
        w.T = 64
        w.x = w.x[:64]
        w.topk_idx = w.topk_idx[:64]
        w.topk_weights = w.topk_weights[:64]
    pins.check_ll_matches_contiguous(orc, w)


def test_replicas_on_c5_routing(orc):
    w = mi.config_c5(T=1024, H=64)  # routing of the replica workload at reduced size
    pins.check_replicas(orc, w, 32)


def test_replicas_on_random_routing(orc):
    for s in range(10):
        w = mi.random_case(s, 50, 16, 16, 4, 3, neg_frac=0.1)
        pins.check_replicas(orc, w, 4 * (s % 3))


def test_bad_ids_and_overflow_status(orc):
    w = mi.random_case(9, 40, 8, 8, 2, 4, bad_frac=0.2)
    lay = orc.layout(w.topk_idx, 8, 2, 1)
    assert lay["status"] & 1
    bad = (w.topk_idx < -1) | (w.topk_idx >= 8)
    assert np.all(lay["slot"][bad] == -1)
    dup = np.zeros((8, 2), np.int64)  # 16 pairs on expert 0, M = 8
    ll = orc.ll_layout(dup, 4, 2, 8, 1)
    assert ll["status"] == 2 and ll["recv_count"][0] == 8
    assert (ll["slot"] >= 0).sum() == 8


def test_empty_batch(orc):
    idx = np.zeros((0, 8), np.int64)
    lay = orc.layout(idx, 256, 8, 4)
    assert lay["rows"] == 0 and lay["count"].sum() == 0 and lay["offset"].sum() == 0
    assert lay["rank_token_count"].sum() == 0


def test_fp8_golden_hand_worked(orc):
    pins.check_fp8_golden(orc)


def test_e4m3_values_match_torch(orc):
    pins.check_e4m3_values_vs_torch(orc)


def test_e4m3_rounding_matches_torch(orc):
    pins.check_e4m3_vs_torch(orc)


def test_fp8_cast_closed_forms(orc):
    pins.check_fp8_cast_on_inputs(orc, n=8)


@pytest.mark.parametrize("flags", [0, 1, 3])
def test_fp8_cast_at_low_latency_config(orc, flags):
    w = mi.config_c3(128)
    pins.check_quantize_properties(orc, w.x, flags)


def test_ll_fp8_dispatch_placement(orc):
    pins.check_ll_fp8_dispatch(orc, n=12)


def test_fp8_tuple_dispatch_is_row_copy(orc):
    """Buffer.dispatch with an (E4M3, scales) tuple: codes and scales land on
    the pair's row, bit for bit, by numpy indexing."""
    w = mi.config_c1()
    qz = orc.quantize_fp8(np.repeat(w.x, 1, axis=1)[:, :256], 0)
    lay = orc.layout(w.topk_idx, w.E, w.R, 4)
    rq, rs, st = orc.dispatch_fp8_tuple(qz["q"], qz["scale"], lay["slot"], lay["rows"],
                                        fill16=0x7E57)
    assert st == 0
    used = np.zeros(lay["rows"], bool)
    for t in range(w.T):
        for k in range(w.K):
            r = lay["slot"][t, k]
            used[r] = True
            assert np.array_equal(rq[r], qz["q"][t]) and np.array_equal(rs[r], qz["scale"][t])
    assert np.all(rq[~used] == 0x57) or np.all(rq[~used].view(np.uint16) == 0x7E57)
    assert np.all(rs[~used].view(np.uint32) == 0x7E577E57)


def test_masked_combine_vs_dense_and_closed_forms(orc):
    pins.check_combine_masked(orc, n=40)


def test_recv_stats_accumulate(orc):
    pins.check_recv_stats(orc)


def test_rank_layout_golden(orc):
    pins.check_rank_golden(orc)


def test_rank_layout_vs_bruteforce(orc):
    pins.check_rank_layout_vs_bruteforce(orc, n=200)


@pytest.mark.parametrize("name,A", [("c1", 1), ("c2", 1), ("c2", 32), ("c4", 1), ("c5", 16)])
def test_rank_layout_closed_forms(orc, name, A):
    w = mi.by_name(name)
    if name == "c5":  # the replica workload's routing, at reduced width
        w = mi.config_c5(T=2048, H=64)
    pins.check_rank_closed_forms(orc, w, A)


def test_replica_weight_sync_and_grad_reduce(orc):
    pins.check_replica_sync_and_reduce(orc)
