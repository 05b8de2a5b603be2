"""The folded stochastic-rounding quantizer's identity, on the CPU in float32.

Stochastic rounding needs floor(-Y) for Y = fl(a * r) * 2^16, where a = |x|
and r = fl(qmax / A) is the block's reciprocal.  For blocks whose r is 0 or
lies in (1/2, 2^100], the kernel multiplies once by r' = r * -2^16 instead
of twice.  These tests check the identity that this relies on, in numpy
float32 arithmetic (IEEE, correctly rounded, subnormals kept):
floor(fl(a * r') ) == floor(fl(fl(a * r) * -2^16)), the same with the first
moment's clamp to qmax, over random and boundary operands, and that r = 1/2
is outside the range (one subnormal a gives a different floor there).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

F = np.float32
NEG16 = F(-65536.0)


def unfolded(a, r, qmax=None):
    y = a * r
    if qmax is not None:
        y = np.minimum(y, F(qmax))
    return np.floor(y * NEG16)


def folded(a, r, qmax=None):
    y = a * (r * NEG16)
    if qmax is not None:
        y = np.maximum(y, F(qmax) * NEG16)
    return np.floor(y)


def in_fold_range(r):
    b = np.asarray(r, dtype=F).view(np.uint32)
    return (b == 0) | ((b > 0x3F000000) & (b <= 0x71800000))


def magnitudes(rng, n):
    """|x| over the float32 range: normals of every exponent, subnormals, 0."""
    e = rng.integers(-150, 12, n)
    a = (rng.random(n) + 0.5) * np.exp2(e.astype(np.float64))
    a = a.astype(F)
    k = rng.integers(1, 2 ** 23, n // 8).astype(np.float64)
    sub = (k * 2.0 ** -149).astype(F)  # subnormals, exact
    return np.concatenate([a, sub, np.array([0.0, 2.0 ** -149, 2.0 ** -126], dtype=F)])


def reciprocals(rng, n):
    """r = qmax / A over the fold range, log-uniform, plus its edges."""
    r = np.exp2(rng.uniform(-1.0, 100.0, n)).astype(F)
    edges = np.array([np.nextafter(F(0.5), F(1)), 1.0, 127.0, 255.0, 2.0 ** 100,
                      np.nextafter(F(2.0 ** 100), F(0)), 0.0], dtype=F)
    return np.concatenate([r[in_fold_range(r)], edges])


@pytest.mark.parametrize("qmax", [None, 127])
def test_folded_floor_equals_the_unfolded_one(qmax):
    rng = np.random.default_rng(5)
    a = magnitudes(rng, 1 << 20)
    r = reciprocals(rng, 1 << 20)
    rr = np.resize(r, a.size)
    assert in_fold_range(rr).all()
    # the values a quantizer meets: a * r at most ~qmax unless clamped
    keep = (a.astype(np.float64) * rr.astype(np.float64) <= 300.0) | (qmax is not None)
    a, rr = a[keep], rr[keep]
    assert np.array_equal(folded(a, rr, qmax), unfolded(a, rr, qmax))
    # every edge reciprocal against every subnormal and tiny normal
    tiny = np.concatenate([(np.arange(1, 4097, dtype=np.float64) * 2.0 ** -149).astype(F),
                           np.exp2(np.arange(-149, -100, dtype=np.float64)).astype(F)])
    for x in r[-7:]:
        assert np.array_equal(folded(tiny, x, qmax), unfolded(tiny, x, qmax)), x


def test_products_beyond_the_range_agree_after_the_clamp():
    # percentile and kept scales let a exceed A: with the clamp both forms
    # give floor(-qmax * 2^16), also where a * r' overflows to -inf
    a = np.array([1e3, 1e20, 3.4e38], dtype=F)
    for r in (F(1.0), F(2.0 ** 100)):
        assert np.array_equal(folded(a, r, 127), unfolded(a, r, 127))
        assert (folded(a, r, 127) == -127 * 65536).all()


def test_half_is_outside_the_range():
    # a = 2^-149, r = 1/2: fl(a * r) ties to 0 (floor 0) while a * r * -2^16
    # is a small normal (floor -1) -- the reason the lower bound is strict
    a, r = F(2.0 ** -149), F(0.5)
    assert unfolded(a, r) == 0.0 and folded(a, r) == -1.0
    assert not in_fold_range(r)
    # beyond 2^112 the folded reciprocal overflows
    assert np.isinf(F(2.0 ** 113) * NEG16)
    assert not in_fold_range(F(2.0 ** 101))
