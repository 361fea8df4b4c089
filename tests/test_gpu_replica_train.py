"""Parity with the oracle of the replica weight sync and the replica gradient
reduction (ultraep GPU operations: Replica weight sync, Replica gradient
reduction). Bar: bit-exact (a bit copy; one float add per element)."""
import numpy as np
import pytest
import torch

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


PLANS = [  # (E, R, C, S, seed)
    (16, 4, 4, 8, 1),
    (16, 4, 4, 1032, 2),
    (64, 8, 16, 4096, 3),
    (8, 2, 0, 64, 4),
    (32, 8, 32, 200, 5),
    (256, 8, 32, 7168 * 64, 6),  # the replica workload's plan, 458752 parameters per expert
]


@pytest.mark.parametrize("plan_case", PLANS)
def test_weight_sync_and_grad_reduce(capi, orc, plan_case):
    E, R, C, S, seed = plan_case
    rng = np.random.default_rng(seed)
    load = rng.integers(0, 1000, E).astype(np.int32)
    plan = orc.plan_replicas(load, R, C)
    Ep = plan["E_phys"]
    rc = to_dev(plan["replica_count"])
    rp = to_dev(plan["replica_phys"].reshape(-1))
    _announce(f"replica sync/reduce E={E} R={R} C={C} S={S}")
    w = rng.integers(0, 1 << 16, (Ep, S)).astype(np.uint16)
    wd = to_dev(w)
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    capi.moe_replica_weight_sync(E, Ep, S, rc, rp, wd, st)
    g = rng.standard_normal((Ep, S)).astype(np.float32)
    gd = to_dev(g)
    capi.moe_replica_grad_reduce(E, Ep, S, rc, rp, gd, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    want_w = orc.replica_weight_sync(w, plan["replica_count"], plan["replica_phys"])
    assert np.array_equal(wd.cpu().numpy().view(np.uint16), want_w)
    want_g = orc.replica_grad_reduce(g, plan["replica_count"], plan["replica_phys"])
    assert np.array_equal(gd.cpu().numpy().view(np.uint32), want_g.view(np.uint32))


def test_bad_replica_entry_is_flagged(capi, orc):
    plan = orc.plan_replicas(np.arange(16, dtype=np.int32), 4, 4)
    rp = plan["replica_phys"].copy()
    hot = int(np.nonzero(plan["replica_count"] == 2)[0][0])
    rp[hot, 1] = 10 ** 6
    w = np.zeros((plan["E_phys"], 16), np.uint16)
    wd = to_dev(w)
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    _announce("replica sync with a bad table entry")
    capi.moe_replica_weight_sync(16, plan["E_phys"], 16, to_dev(plan["replica_count"]),
                                 to_dev(rp.reshape(-1)), wd, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 8


def test_sync_twice_then_reduce(capi, orc):
    """A second sync after the masters changed copies the new masters."""
    E, R, C, S = 16, 4, 8, 256
    plan = orc.plan_replicas(np.arange(E, dtype=np.int32)[::-1].copy(), R, C)
    Ep = plan["E_phys"]
    rng = np.random.default_rng(7)
    w = rng.integers(0, 1 << 16, (Ep, S)).astype(np.uint16)
    wd = to_dev(w)
    rc, rp = to_dev(plan["replica_count"]), to_dev(plan["replica_phys"].reshape(-1))
    _announce("replica sync twice")
    capi.moe_replica_weight_sync(E, Ep, S, rc, rp, wd)
    prim = plan["replica_phys"][:, 0]
    w2 = wd.cpu().numpy().view(np.uint16).copy()
    w2[prim] = rng.integers(0, 1 << 16, (E, S)).astype(np.uint16)
    wd.copy_(to_dev(w2))
    capi.moe_replica_weight_sync(E, Ep, S, rc, rp, wd)
    torch.cuda.synchronize()
    assert np.array_equal(wd.cpu().numpy().view(np.uint16),
                          orc.replica_weight_sync(w2, plan["replica_count"],
                                                  plan["replica_phys"]))
