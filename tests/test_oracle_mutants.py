"""Each planted mistake in the oracle (built with -DORACLE_MUTANT=n) must be
caught by at least one pin, so the pins are not vacuous."""
import os

import pytest

import oracle
import pins

MUTANTS = {
    1: "alignment dropped from the offset scan",
    2: "pairs ranked in column-major order",
    3: "last top-k term dropped from combine",
    4: "weight index reversed in combine",
    5: "per-rank count counts pairs, not distinct tokens",
    6: "low-latency row drops the source stripe",
    7: "replicas planned for the coldest experts",
    8: "replica chosen by k instead of by token",
    9: "bf16 rounding ties away from even",
    10: "E4M3 rounding ties away from zero",
    11: "FP8 scale from the FNUZ maximum 240",
    12: "round_scale rounds the scale down",
    13: "low-latency FP8 scales stored row-major",
    14: "UE8M0 bytes packed high to low",
    15: "FP8 amax over the whole row",
    16: "row-major UE8M0 scales stored transposed",
    17: "masked combine takes the rank as e mod R",
    18: "normal-mode rows in descending token order",
    19: "normal-mode received ids global instead of rank-local",
    20: "replica gradient replaces the master gradient",
}


def _run_all(orc):
    import moe_inputs as mi

    failures = []
    checks = list(pins.ALL_SMALL_CHECKS) + [
        lambda o: pins.check_bf16_vs_torch(o, n=1 << 16),
        lambda o: pins.check_replicas(o, mi.random_case(3, 50, 16, 16, 4, 3, neg_frac=0.1), 4),
        lambda o: pins.check_layout_invariants(o, mi.config_c1(), 16),
    ]
    for chk in checks:
        try:
            chk(orc)
        except AssertionError:
            failures.append(getattr(chk, "__name__", "lambda"))
    return failures


def test_normal_build_passes_all(orc):
    assert orc.mutant == 0
    assert _run_all(orc) == []


@pytest.mark.parametrize("n", sorted(MUTANTS))
def test_mutant_is_caught(n, tmp_path):
    path = os.path.join(str(tmp_path), f"liboracle_m{n}.so")
    oracle.build(path, mutant=n)
    orc = oracle.Oracle(path)
    assert orc.mutant == n
    assert _run_all(orc), f"mutant {n} ({MUTANTS[n]}) slipped past every pin"
