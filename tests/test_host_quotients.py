"""Host check of the exactly rounded quotients the RMS / Hadamard kernels take
from reciprocal products (x / r in fp32 and y / sqrt(128) rounded to fp32).

The kernels form z = RN64(x * RN64(1 / r)), within 2 fp64 units in the last
place of the quotient, round z to fp32, and divide outright only when z lies
within 8 fp64 units of an fp32 rounding midpoint of its binade (or below the
fp32 normal range).  This test emulates that decision in numpy: it pins the
bit test against constructed values on both sides of a midpoint, and checks on
random inputs that every product it trusts rounds to the correctly rounded
quotient (a double rounding through fp64 is exact for fp32 operands: 53 >=
2 * 24 + 2)."""
import numpy as np


def unsure(z):
    """The kernels' test: low 29 bits of the fp64 pattern within 8 of 2^28
    (an fp32 midpoint), or a nonzero value below 2^-125."""
    lo = z.view(np.uint64).astype(np.uint64) & np.uint64(0xFFFFFFFF)
    mid = ((lo + np.uint64(8) - np.uint64(0x10000000)) & np.uint64(0x1FFFFFFF)) <= np.uint64(16)
    return mid | ((np.abs(z) < 2.0 ** -125) & (z != 0.0))


def test_flag_window_around_midpoints():
    rng = np.random.default_rng(5)
    f = rng.uniform(1.0, 2.0, 2000).astype(np.float32)
    # the fp32 midpoint above f: f + ulp32 / 2, exact in fp64
    m = f.astype(np.float64) + np.ldexp(1.0, np.frexp(f.astype(np.float64))[1] - 25)
    for k in range(-8, 9):
        z = m + k * np.ldexp(1.0, np.frexp(m)[1] - 53)
        assert unsure(z).all(), k
    for k in (-40, -12, 12, 40):
        z = m + k * np.ldexp(1.0, np.frexp(m)[1] - 53)
        assert not unsure(z).any(), k
    assert not unsure(f.astype(np.float64)).any()          # fp32 values themselves
    assert unsure(np.array([2.0 ** -130, -2.0 ** -126])).all()  # below the fp32 normal range
    assert not unsure(np.array([0.0])).any()


def test_trusted_products_round_like_the_division():
    rng = np.random.default_rng(6)
    n = 400_000
    # bf16-valued inputs over a wide exponent range, and their RMS-like divisors
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    r = np.abs(rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32) + np.float32(1e-30)
    inv = 1.0 / r.astype(np.float64)
    z = x.astype(np.float64) * inv
    exact = (x.astype(np.float64) / r.astype(np.float64)).astype(np.float32)
    ok = ~unsure(z)
    assert np.array_equal(z[ok].astype(np.float32).view(np.uint32), exact[ok].view(np.uint32))
    # y / sqrt(128): y an fp64 butterfly output, the reference rounds twice
    y = rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n)) * (1.0 + rng.random(n))
    rs = np.sqrt(128.0)
    w = y * (1.0 / rs)
    ref = (y / rs).astype(np.float32)
    ok = ~unsure(w)
    assert np.array_equal(w[ok].astype(np.float32).view(np.uint32), ref[ok].view(np.uint32))
    assert ok.mean() > 0.999  # the division is the rare path
