"""The kernels find the token of a wave or workgroup b as (b * m) >> 32 with
m = ceil(2^32 / d) (d: waves or workgroups per token), wherever the host has
checked that every b in the grid satisfies b * d < 2^32 (and divide
otherwise). That claim, checked here on the CPU with exact integers: every
b below the bound gives floor(b / d), for divisors from 1 to 4096 and the
row widths the library takes, exhaustively near 0 and at the bound, where
the error of the reciprocal is largest."""
import random


def magic(d):
    return ((1 << 32) + d - 1) // d


def quotient(b, m):
    return (b * m) >> 32


def _bound(d):
    return ((1 << 32) - 1) // d  # the largest b with b * d < 2^32


def _check(d, bs):
    m = magic(d)
    for b in bs:
        assert quotient(b, m) == b // d, (d, b)


def test_small_divisors_exhaustive_near_zero_and_bound():
    for d in range(1, 257):
        n = _bound(d)
        _check(d, range(0, min(n, 4096) + 1))
        _check(d, range(max(0, n - 4096), n + 1))


def test_row_chunk_divisors():
    # chunks per token row: 1 KiB chunks (the scatter and the fused kernels,
    # 16-byte lanes) and 512 B (the combine, 8-byte lanes) for H = 8..2^20
    rng = random.Random(5)
    ds = set()
    for H in [8, 256, 1000, 4096, 7168, 1 << 16, 1 << 20] + [8 * rng.randrange(1, 1 << 17)
                                                           for _ in range(40)]:
        for lane_bytes in (16, 8):
            ds.add(-(-H * 2 // lane_bytes // 64))
    for d in sorted(ds):
        n = _bound(d)
        _check(d, range(max(0, n - 2000), n + 1))
        _check(d, [rng.randrange(0, n + 1) for _ in range(2000)])


def test_a_bound_is_needed():
    # the bound is sufficient, not tight; but some bound is needed: for d = 3
    # (m = (2^32 + 2) / 3) the reciprocal's error b * (2/3) / 2^32 reaches, at
    # b = 2^31, the 1/3 that b mod 3 = 2 leaves below the next integer, and
    # the quotient comes out one too high -- which is why the host divides for
    # grids that reach past b * d < 2^32
    d = 3
    m = magic(d)
    assert all(quotient(b, m) == b // d for b in range((1 << 31) - 64, 1 << 31))
    assert quotient(1 << 31, m) == (1 << 31) // d + 1
