"""Sanity of the seeded workload generators (shapes, determinism, the
statistics the recipes imply). Not parity: no method arithmetic is here."""
import numpy as np

import moe_inputs as mi


def test_shapes_and_determinism():
    for f in (mi.config_c1, mi.config_c2):
        a, b = f(), f()
        assert np.array_equal(a.x, b.x) and np.array_equal(a.topk_idx, b.topk_idx)
        assert a.x.shape == (a.T, a.H) and a.x.dtype == np.uint16
        assert a.topk_idx.shape == (a.T, a.K) and a.topk_idx.dtype == np.int64
        assert a.topk_weights.shape == (a.T, a.K) and a.topk_weights.dtype == np.float32
        assert np.allclose(a.topk_weights.sum(1), 1, atol=1e-6)


def test_c2_uniform_routing_statistics():
    w = mi.config_c2()
    ids = w.topk_idx
    assert all(len(set(r)) == w.K for r in ids.tolist())  # distinct experts per token
    cnt = np.bincount(ids.ravel(), minlength=w.E)
    assert cnt.sum() == 1024 and abs(cnt.mean() - 4) < 1e-9 and cnt.max() <= 16
    ranks = np.zeros((w.T, w.R), bool)
    ranks[np.repeat(np.arange(w.T), w.K), (ids // w.L).ravel()] = True
    # E[tokens per rank] = T * (1 - C(224,8)/C(256,8)) ~ 84.7
    assert 70 < ranks.sum(0).mean() < 100


def test_zipf_skew():
    w = mi.config_c4()
    assert all(len(set(r)) == w.K for r in w.topk_idx[:512].tolist())
    cnt = np.bincount(w.topk_idx.ravel(), minlength=w.E)
    assert cnt.max() > 8 * cnt.mean()  # hottest expert ~ 9.7x the mean
    perm = w.meta["perm"]
    assert cnt[perm[0]] == cnt.max()


def test_c3_sweep_shapes():
    for M in mi.C3_SWEEP[:3]:
        w = mi.config_c3(M)
        assert w.T == M and w.M == M and w.H == 7168 and w.E == 256 and w.K == 8
