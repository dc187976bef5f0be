"""Property tests of the oracle (CPU, hypothesis): invariants that must hold for any input, drawn at
random, against definitions written out here independently of the oracle's code paths (exact
rationals, brute-force loops, nearest-value searches)."""
from fractions import Fraction

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from hypothesis.extra.numpy import arrays

import oracle as O

F32 = np.float32
SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])

# zero, or magnitudes in [2^-100, 2^20]: a row's step stays a normal binary32 number, where the
# quantiser's invariants hold
finite32 = st.one_of(st.just(0.0), st.floats(2.0 ** -100, 2.0 ** 20, width=32),
                     st.floats(-(2.0 ** 20), -(2.0 ** -100), width=32))
rows = arrays(np.float32, st.tuples(st.integers(1, 4), st.integers(1, 96)), elements=finite32)


def rne_fraction(q: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


@SETTINGS
@given(rows)
def test_quantize_rows_codes_are_rne_of_exact_quotients(y):
    """Each code is round-half-even of fl32(y / step), clipped; step = fl32(absmax / 127)."""
    q, step = O.quantize_rows(y)
    for r in range(y.shape[0]):
        amax = float(np.max(np.abs(y[r])))
        assert step[r] == F32(amax) / F32(127)
        if step[r] == 0:
            assert not q[r].any()
            continue
        for v, c in zip(y[r], q[r]):
            t = F32(v) / step[r]                                  # the binary32 quotient the method rounds
            want = max(-127, min(127, rne_fraction(Fraction(float(t)))))
            assert int(c) == want


@SETTINGS
@given(rows)
def test_quantize_rows_invariants(y):
    q, step = O.quantize_rows(y)
    qn, stepn = O.quantize_rows(-y)
    assert np.array_equal(stepn, step) and np.array_equal(qn, -q)          # odd symmetry
    for r in range(y.shape[0]):
        if step[r] == 0:
            continue
        assert np.max(np.abs(q[r].astype(np.int64))) == 127                    # the row max reaches 127
        err = np.abs(q[r].astype(np.float64) * float(step[r]) - y[r].astype(np.float64))
        assert np.all(err <= float(step[r]) / 2 * (1 + 2.0 ** -15))
        order = np.argsort(y[r], kind="stable")
        assert np.all(np.diff(q[r][order].astype(np.int64)) >= 0)             # monotone in y


@SETTINGS
@given(st.lists(st.integers(-126, 126), min_size=1, max_size=40), st.integers(0, 1))
def test_quantize_rows_ties_go_to_even(ks, sign):
    """A row whose absmax is 127 has step exactly 1, so k + 1/2 lands on a tie."""
    vals = [k + 0.5 for k in ks] + [127.0 if sign else -127.0]
    q, step = O.quantize_rows(np.array([vals], F32))
    assert step[0] == 1.0
    for v, c in zip(vals[:-1], q[0][:-1]):
        lo = int(np.floor(v))
        assert int(c) == (lo if lo % 2 == 0 else lo + 1)


@SETTINGS
@given(rows)
def test_quantize_tensor_is_the_rows_quantiser_with_one_step(y):
    q, step = O.quantize_tensor(y)
    amax = float(np.max(np.abs(y)))
    assert np.all(step == F32(amax) / F32(127))
    if amax:
        assert np.max(np.abs(q.astype(np.int64))) == 127
        for v, c in zip(y.ravel(), q.ravel()):
            t = F32(v) / F32(step.ravel()[0])
            assert int(c) == max(-127, min(127, rne_fraction(Fraction(float(t)))))


@SETTINGS
@given(st.integers(1, 40), st.integers(1, 40), st.sampled_from([64, 128, 192, 256]), st.integers(0, 2 ** 32 - 1))
def test_int_gemm_equals_integer_loops(m, n, k, seed):
    rng = np.random.default_rng(seed)
    xq = rng.integers(-127, 128, (m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, (n, k), dtype=np.int8)
    acc = O.int_gemm(xq, wq)
    i, j = rng.integers(0, m), rng.integers(0, n)
    assert acc[i, j] == sum(int(a) * int(b) for a, b in zip(xq[i], wq[j]))
    assert np.array_equal(acc, xq.astype(np.int64) @ wq.astype(np.int64).T)


E4M3_GRID = np.sort(np.unique(np.abs(O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64))))


@SETTINGS
@given(arrays(np.float32, st.integers(1, 64), elements=st.floats(-448, 448, width=32, allow_nan=False)))
def test_e4m3_encode_picks_the_nearest_value_ties_to_even(v):
    codes = O.e4m3_encode(v)
    dec = np.abs(O.e4m3_decode(codes).astype(np.float64))
    a = np.abs(v.astype(np.float64))
    for x, d, c in zip(a, dec, codes):
        i = np.searchsorted(E4M3_GRID, x)
        cands = E4M3_GRID[max(0, i - 1):i + 1]
        best = np.min(np.abs(cands - x))
        assert abs(d - x) == best                                     # nearest representable magnitude
        near = cands[np.abs(cands - x) == best]
        if len(near) == 2:                                            # a tie: the even mantissa (code bit 0 clear)
            assert (int(c) & 1) == 0


@SETTINGS
@given(arrays(np.float32, st.integers(1, 32), elements=st.floats(2.0 ** -10, 1024.0, width=32)),
       arrays(np.float32, st.integers(1, 32), elements=st.floats(2.0 ** -10, 1024.0, width=32)))
def test_alpha_half_balances_the_smoothed_maxima(a, w):
    k = min(len(a), len(w))
    a, w = a[:k], w[:k]
    s, _, _ = O.smoothing_factors(a, w, 0.5)
    s64 = s.astype(np.float64)
    # at alpha = 0.5 the smoothed activation max a/s and weight max w*s both equal sqrt(a w), up to s's rounding
    gm = np.sqrt(a.astype(np.float64) * w.astype(np.float64))
    assert np.allclose(a / s64, gm, rtol=2.0 ** -22)
    assert np.allclose(w * s64, gm, rtol=2.0 ** -22)


@SETTINGS
@given(st.integers(1, 6), st.integers(1, 6), st.integers(1, 24), st.floats(0.0, 1.0), st.integers(0, 2 ** 32 - 1))
def test_fold_preserves_the_product_in_binary64(m, n, k, alpha, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)) * np.where(rng.random(k) < 0.2, 50.0, 1.0)
    w = rng.standard_normal((n, k)) * 0.02
    a = np.max(np.abs(x), axis=0).astype(F32)
    s, _, _ = O.smoothing_factors(a, O.weight_colmax(w.astype(F32), "f32"), alpha)
    s64 = s.astype(np.float64)
    lhs = x @ w.T
    rhs = (x / s64) @ (w * s64).T
    assert np.allclose(rhs, lhs, rtol=1e-12, atol=1e-12 * np.max(np.abs(lhs)))
