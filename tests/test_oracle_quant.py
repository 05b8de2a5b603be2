"""Pins for the oracle's block statistic, codebook and quantizer.

Each check compares against something other than the oracle's own formula:
brute-force nearest-code search over the whole alphabet, exhaustive
enumeration of all 2^16 stochastic-rounding draws against a closed-form
count, numpy.percentile(method="lower"), a brute maximum, and properties
that must hold for any correct block quantizer with the reading taken here
(round trip within half a step, exact constant blocks, dequantize ->
requantize fixed point).
"""
import numpy as np
import pytest

U = 2.0 ** -24  # fp32 unit roundoff


def _ulp(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


# -------------------------------------------------------------- statistic
@pytest.mark.parametrize("n", [1, 2, 16, 17, 1000, 1792, 2047, 2048])
def test_absmax_is_brute_max(orc, n):
    rng = np.random.default_rng(n)
    a = np.abs(rng.standard_normal(n).astype(np.float32))
    assert orc.block_stat(a) == float(np.max(a))


@pytest.mark.parametrize("p", [0.0, 12.5, 50.0, 93.75, 99.0, 99.9, 100.0, 37.3, 0.1])
@pytest.mark.parametrize("n", [1, 2, 5, 16, 1000, 1792, 2047, 2048])
def test_percentile_matches_numpy_lower(orc, p, n):
    rng = np.random.default_rng([n, int(p * 100)])
    a = (np.abs(rng.standard_normal(n)) + 1e-3).astype(np.float32)
    p32 = np.float32(p)
    want = np.percentile(a, np.float64(p32), method="lower")
    assert orc.block_stat(a, use_pct=True, p=float(p32)) == float(want)
    assert orc.percentile_rank(float(p32), n) == int(np.searchsorted(np.sort(a), want))


def test_percentile_100_is_absmax(orc):
    rng = np.random.default_rng(3)
    for n in [1, 7, 2048]:
        a = np.abs(rng.standard_normal(n)).astype(np.float32)
        assert orc.block_stat(a, True, 100.0) == orc.block_stat(a)


def test_percentile_rank_at_block_sizes(orc):
    # 99.9th percentile of 2048 is the 4th largest; tails shift it
    assert orc.percentile_rank(99.9, 2048) == 2044
    assert orc.percentile_rank(99.9, 1792) == 1789
    assert orc.percentile_rank(99.9, 1000) == 998
    assert orc.percentile_rank(0.0, 2048) == 0
    assert orc.percentile_rank(100.0, 2048) == 2047


def test_percentile_zero_falls_back_to_max(orc):
    a = np.zeros(2048, np.float32)
    a[5] = 3.0
    assert orc.block_stat(a, True, 50.0) == 3.0


# -------------------------------------------------------------- quantizer
@pytest.mark.parametrize("signed", [True, False])
def test_rne_codes_are_nearest_in_alphabet(orc, signed):
    rng = np.random.default_rng(5 + signed)
    qmax = 127 if signed else 255
    alphabet = np.arange(-qmax if signed else 0, qmax + 1)
    for trial in range(40):
        n = 16
        x = rng.standard_normal(n).astype(np.float32) * np.float32(10.0 ** rng.uniform(-8, 3))
        if not signed:
            x = np.abs(x)
        codes, A = orc.quantize_block(x, signed)
        assert A == np.max(np.abs(x))
        values = orc.dequantize_block(alphabet, signed, float(A)).astype(np.float64)
        dist = np.abs(values[None, :] - x.astype(np.float64)[:, None])
        best = dist.min(axis=1)
        chosen = dist[np.arange(n), codes - alphabet[0]]
        assert np.all(chosen <= best + 4 * U * float(A)), trial


@pytest.mark.parametrize("signed", [True, False])
def test_round_trip_within_half_step(orc, signed):
    rng = np.random.default_rng(17 + signed)
    qmax = 127 if signed else 255
    for trial in range(30):
        n = int(rng.integers(1, 2049))
        x = rng.standard_normal(n).astype(np.float32) * np.float32(10.0 ** rng.uniform(-12, 4))
        if not signed:
            x = x * x
        codes, A = orc.quantize_block(x, signed)
        back = orc.dequantize_block(codes, signed, float(A)).astype(np.float64)
        err = np.abs(back - x)
        assert np.all(err <= float(A) / (2 * qmax) + 2 * _ulp(A)), trial
        assert codes.min() >= (-qmax if signed else 0) and codes.max() <= qmax


@pytest.mark.parametrize("signed", [True, False])
@pytest.mark.parametrize("stochastic", [False, True])
def test_constant_blocks_round_trip_exactly(orc, signed, stochastic):
    rng = np.random.default_rng(23)
    cs = list(rng.standard_normal(200).astype(np.float32) * np.float32(10.0) ** rng.uniform(
        -30, 30, 200).astype(np.float32)) + [np.float32(1.0), np.float32(1e-30), np.float32(3e38)]
    for c in cs:
        c = np.float32(c if signed else abs(c))
        x = np.full(37, c, np.float32)
        draws = rng.integers(0, 1 << 16, 37).astype(np.uint16) if stochastic else None
        codes, A = orc.quantize_block(x, signed, draws=draws)
        back = orc.dequantize_block(codes, signed, float(A))
        assert np.array_equal(back, x), c
    zero = np.zeros(9, np.float32)
    codes, A = orc.quantize_block(zero, signed)
    assert A == 0 and not codes.any()
    assert not orc.dequantize_block(codes, signed, float(A)).any()


@pytest.mark.parametrize("signed", [True, False])
def test_dequantize_requantize_fixed_point(orc, signed):
    qmax = 127 if signed else 255
    alphabet = np.arange(-qmax if signed else 0, qmax + 1)
    rng = np.random.default_rng(29)
    As = list(np.float32(10.0) ** rng.uniform(-33, 37, 300).astype(np.float32)) + [
        np.float32(1.0), np.float32(2.0 ** -112), np.float32(3.4e38)]
    for A in As:
        x = orc.dequantize_block(alphabet, signed, float(A))
        codes, A2 = orc.quantize_with_stat(x, signed, float(A))
        assert A2 == np.float32(A)
        assert np.array_equal(codes, alphabet), A


@pytest.mark.parametrize("signed", [True, False])
def test_stochastic_rounding_counts_over_all_draws(orc, signed):
    # With A = qmax the reciprocal scale is exactly 1, so y = |x| exactly and
    # the number of the 2^16 draws that round up must be ceil(frac * 2^16).
    qmax = 127 if signed else 255
    draws = np.arange(1 << 16, dtype=np.uint16)
    vals = [5.25, 2.1, 0.0001, 126.99999, 0.5, 3.0, 77.123456]
    for a in vals:
        a32 = np.float32(a)
        x = np.full(1 << 16, -a32 if signed else a32, np.float32)
        codes, _ = orc.quantize_with_stat(x, signed, float(qmax), draws=draws)
        k = np.abs(codes)
        lo = int(np.floor(np.float64(a32)))
        frac = np.float64(a32) - lo
        assert set(np.unique(k)).issubset({lo, lo + 1})
        assert int((k == lo + 1).sum()) == int(np.ceil(frac * 65536)), a
        # the endpoint pins to qmax regardless of the draw
    x = np.full(16, np.float32(qmax), np.float32)
    codes, _ = orc.quantize_with_stat(x, signed, float(qmax), draws=draws[:16])
    assert np.all(np.abs(codes) == qmax)


def test_stochastic_rounding_is_unbiased_over_seeds(orc):
    # mean of the dequantized value over independent Philox draws -> x
    x = np.array([0.123, -0.77, 0.5004, -0.999, 0.0101, 1.0, -0.3333, 0.9],
                 np.float32)
    acc = np.zeros(x.size)
    trials = 3000
    for s in range(trials):
        d = orc.sr_draws(s, 1, 0, x.size, 0)
        codes, A = orc.quantize_block(x, True, draws=d)
        acc += orc.dequantize_block(codes, True, float(A))
    mean = acc / trials
    step = 1.0 / 127
    assert np.all(np.abs(mean - x) < 5 * step * 0.5 / np.sqrt(trials) + 1e-6)


def test_signed_codes_never_use_minus_128(orc):
    rng = np.random.default_rng(31)
    x = -np.abs(rng.standard_normal(2048).astype(np.float32))
    codes, _ = orc.quantize_block(x, True)
    assert codes.min() == -127


def test_tiny_block_statistic_encodes_zero(orc):
    x = np.full(8, np.float32(2.0 ** -120), np.float32)
    codes, A = orc.quantize_block(x, True)
    assert A == 0 and not codes.any()


# -------------------------------------------------------------- exact ties
# Reading S8 (nearest rounding breaks ties to even; the 8-bit Adam page names
# only the stochastic option, so deterministic ties are a reading): a block
# whose statistic is A = qmax * 2^e has r = fl(qmax / A) = 2^-e exactly, so an
# element of magnitude (k + 1/2) * 2^e lands on y = k + 1/2 with no rounding
# at all, and its code must be the even one of k and k + 1.  A quantizer that
# rounds half away from zero (or half up) differs on every odd k.
@pytest.mark.parametrize("signed", [True, False])
@pytest.mark.parametrize("e", [-100, -20, -3, 0, 7, 40])
def test_nearest_rounding_ties_go_to_even(orc, signed, e):
    qmax = 127 if signed else 255
    scale = np.float32(2.0 ** e)
    k = np.arange(qmax, dtype=np.int64)                  # 0 .. qmax-1
    mags = (k.astype(np.float32) + np.float32(0.5)) * scale  # exact
    want = np.where(k % 2 == 0, k, k + 1)                 # the even neighbour
    if signed:
        x = np.concatenate([mags, -mags, [np.float32(qmax) * scale]]).astype(np.float32)
        want_codes = np.concatenate([want, -want, [qmax]])
    else:
        x = np.concatenate([mags, [np.float32(qmax) * scale]]).astype(np.float32)
        want_codes = np.concatenate([want, [qmax]])
    # the statistic found in the block (its maximum) and the one given
    codes, A = orc.quantize_block(x, signed)
    assert A == np.float32(qmax) * scale
    assert np.array_equal(codes, want_codes)
    codes2, _ = orc.quantize_with_stat(x, signed, float(np.float32(qmax) * scale))
    assert np.array_equal(codes2, want_codes)
    # the percentile statistic at 100 is the same maximum
    codes3, _ = orc.quantize_block(x, signed, use_pct=True, p=100.0)
    assert np.array_equal(codes3, want_codes)


def test_step_ties_go_to_even(orc):
    # A whole 8-bit step in which the moments land on exact ties: with
    # beta1 = beta2 = 0 the new first moment is the gradient itself and the
    # second moment its square, and the block layout below makes the first
    # moment's y = |m| * fl(127/A) an exact half-integer on every element but
    # the block maximum.
    rng = np.random.default_rng(41)
    n = 2048 + 700
    k = rng.integers(0, 127, n)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    g = (sign * (k + 0.5) * 2.0 ** -12).astype(np.float32)
    g[0] = np.float32(127 * 2.0 ** -12)       # block 0's maximum
    g[2048] = np.float32(-127 * 2.0 ** -12)   # block 1's maximum (ragged block)
    st = orc.OracleState([n], "q8")
    p = [np.zeros(n, np.float32)]
    st.step(p, [g], lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0, t=1,
            decoupled=True, stochastic=False, percentile=None, seed=1)
    codes = st.buffers()["m_codes"][:n].astype(np.int64)
    want = np.where(k % 2 == 0, k, k + 1) * sign.astype(np.int64)
    want[0], want[2048] = 127, -127
    assert np.array_equal(codes, want)
    assert np.array_equal(st.buffers()["m_scale"], np.float32([127 * 2.0 ** -12] * 2))
