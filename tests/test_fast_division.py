"""The prefill kernel divides by launch constants (head-group sizes, H, the GQA
ratio) with a multiply and a shift whose constants the host computes (Granlund
and Montgomery, "Division by invariant integers using multiplication", 1994:
m = ceil(2^(31+l) / d), l = ceil(log2 d), q = (n * m) >> (31 + l) for
0 <= n < 2^31).  The host's recipe, restated here, is checked against integer
division on every divisor up to 4096 and on large ones, at the dividends where
a rounding mistake would show first."""
import random


def div_const(d):
    if d <= 1:
        return 0, 0
    l = 0
    while (1 << l) < d:
        l += 1
    m = ((1 << (31 + l)) + d - 1) // d
    assert m < (1 << 32)
    return m, l - 1


def div_by(n, c):
    m, s = c
    return n if m == 0 else ((n * m) >> 32) >> s


def _dividends(d, rng):
    top = (1 << 31) - 1
    out = {0, 1, d - 1, d, d + 1, top, top - 1, top - (top % d), top - (top % d) - 1}
    for k in (1, 2, 3, 1000, (top // d) - 1, top // d):
        out.update({k * d - 1, k * d, k * d + 1})
    out.update(rng.randrange(0, top + 1) for _ in range(200))
    return sorted(n for n in out if 0 <= n <= top)


def test_small_divisors():
    rng = random.Random(11)
    for d in range(1, 4097):
        c = div_const(d)
        for n in _dividends(d, rng):
            assert div_by(n, c) == n // d, (n, d)


def test_large_divisors():
    rng = random.Random(12)
    for d in [(1 << k) + e for k in range(12, 31) for e in (-1, 0, 1)] + [rng.randrange(4097, 1 << 31) for _ in range(300)]:
        c = div_const(d)
        for n in _dividends(d, rng):
            assert div_by(n, c) == n // d, (n, d)
