"""Pins of the oracle's near-tie machinery (CPU).

Two oracle functions decide what counts as a correct rounding where an exact
real sits next to a binary32 rounding boundary, and the GPU checks trust them:

* `_s_exact`, the high-precision re-evaluation of a smoothing factor
  s = a^alpha / w^(1 - alpha) ("LLM.int8() and SmoothQuant", "going deeper /
  SmoothQuant"; "SmoothQuant, in depth", "The calibration data flow": the eps
  clamps) that smoothing_factors takes when the binary64 quotient lands within
  2^-16 spacings of a binary32 midpoint. It is pinned here against mpmath at 120
  significant digits, an evaluation that shares no code with it.
* `row_y_variants` / `norm_quant_row_variants`, which list the normalised rows
  (and their codes) for every admissible rounding of a row's mean and variance.
  They are pinned on constructed rows whose statistics sit exactly on, or next
  to, a binary32 midpoint, against closed forms and exact rationals.

Each pin is also shown to catch a planted mistake.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle as O
import oracle.smoothquant_oracle as OM

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------- s near a binary32 midpoint

def _mp_round32(v):
    """Nearest binary32 to the mpmath real v > 0 (ties to even), the distance from v to the
    rounding boundary on v's side in binary32 spacings, and the neighbour past that boundary."""
    e = int(mpmath.floor(mpmath.log(v, 2))) - 23            # spacing 2^e in v's binade (normal range)
    u = v / mpmath.mpf(2) ** e                                # in [2^23, 2^24)
    q = int(mpmath.floor(u))
    frac = u - q
    dist = float(abs(frac - mpmath.mpf(0.5)))
    up = frac > 0.5 or (frac == 0.5 and q % 2 == 1)
    near, far = (q + 1, q) if up else (q, q + 1)
    return F32(near * 2.0 ** e), dist, F32(far * 2.0 ** e)


def _mp_s(a, w, alpha):
    """a^alpha / w^(1 - alpha) at 120 digits, the weight exponent being the binary64 difference 1 - alpha."""
    with mpmath.workdps(120):
        v = mpmath.mpf(float(a)) ** mpmath.mpf(alpha) / mpmath.mpf(float(w)) ** mpmath.mpf(1.0 - alpha)
        return _mp_round32(v)


def _near_midpoint_cases(per_alpha=4):
    """Seeded (a, w, alpha), all binary32 and above the eps clamp, whose binary64 quotient lies within
    2^-16 spacings of a binary32 midpoint. numpy only filters the search; every case is then re-derived
    by the oracle and by mpmath."""
    rng = np.random.default_rng(20240601)
    cases = []
    for alpha in (0.5, 0.65, 0.8, 0.9):
        found = 0
        for _ in range(8):
            n = 1 << 18
            a = (10.0 ** rng.uniform(-3, 3, n)).astype(F32)
            w = (10.0 ** rng.uniform(-4, 0, n)).astype(F32)
            v = np.power(a.astype(F64), alpha) / np.power(w.astype(F64), 1.0 - alpha)
            m, _ = np.frexp(v)                                  # v = m 2^e, m in [0.5, 1)
            u = m * 2.0 ** 24                                   # in binary32 spacings, exact
            dist = np.abs(u - np.floor(u) - 0.5)
            for i in np.where(dist < 2.0 ** -16)[0][: per_alpha - found]:
                cases.append((float(a[i]), float(w[i]), alpha))
                found += 1
            if found >= per_alpha:
                break
    return cases


CASES = _near_midpoint_cases()


def _s_exact_mismatches(fn):
    bad = []
    for a, w, alpha in CASES:
        s, dist, other = fn(a, w, alpha)
        s_m, dist_m, other_m = _mp_s(a, w, alpha)
        if not (F32(s) == s_m and F32(other) == other_m and abs(dist - dist_m) < 1e-9):
            bad.append((a, w, alpha, s, s_m, dist, dist_m))
    return bad


def test_near_midpoint_search_finds_cases():
    assert len(CASES) >= 12
    for a, w, alpha in CASES:
        assert 0 < _mp_s(a, w, alpha)[1] < 2.0 ** -15


def test_s_exact_matches_mpmath_near_midpoints():
    assert _s_exact_mismatches(OM._s_exact) == []


def test_smoothing_factors_take_the_exact_path_near_midpoints(monkeypatch):
    calls = []
    real = OM._s_exact

    def counting(a, w, alpha):
        calls.append((a, w, alpha))
        return real(a, w, alpha)

    monkeypatch.setattr(OM, "_s_exact", counting)
    for a, w, alpha in CASES:
        s, dist, other = O.smoothing_factors([a], [w], alpha)
        s_m, dist_m, other_m = _mp_s(a, w, alpha)
        assert s[0] == s_m and other[0] == other_m and abs(dist[0] - dist_m) < 1e-9
    assert len(calls) >= len(CASES) - 2        # numpy's and libm's pow may disagree on a case or two


def test_s_exact_pin_catches_planted_mistakes():
    from decimal import Decimal, localcontext

    def weight_exponent_alpha(a, w, alpha):
        with localcontext() as ctx:
            ctx.prec = 60
            v = (Decimal(a) ** Decimal(alpha)) / (Decimal(w) ** Decimal(alpha))
        f = Fraction(v)
        return O.rn32_rational(f.numerator, f.denominator)

    def too_few_digits(a, w, alpha):
        with localcontext() as ctx:
            ctx.prec = 10
            v = (Decimal(a) ** Decimal(alpha)) / (Decimal(w) ** Decimal(1.0 - alpha))
        f = Fraction(v)
        return O.rn32_rational(f.numerator, f.denominator)

    def binary64_only(a, w, alpha):
        f = Fraction(pow(a, alpha) / pow(w, 1.0 - alpha))
        return O.rn32_rational(f.numerator, f.denominator)

    for mutant in (weight_exponent_alpha, too_few_digits, binary64_only):
        assert _s_exact_mismatches(mutant), mutant.__name__


# --------------------------------------------------------------------------- statistics on a midpoint

def _mean_midpoint_row():
    """64 values: 32 x 1.0 and 32 x (1 + 2^-23). The mean 1 + 2^-24 is exactly the midpoint of the
    binary32 neighbours 1 and 1 + 2^-23; the variance 2^-48 is a power of two (exact)."""
    return np.array([1.0] * 32 + [1.0 + 2.0 ** -23] * 32, F32)


def test_mean_on_a_midpoint_gives_both_roundings():
    x = _mean_midpoint_row()
    st = O.row_stats(x, O.LAYERNORM)
    assert st["mu"] == F32(1.0) and st["mu_other"] == F32(1.0 + 2.0 ** -23) and st["mu_dist"] == 0.0
    assert st["var"] == F32(2.0 ** -48) and st["var_dist"] == 0.5
    variants = O.norm_quant_row_variants(x, "f32", O.LAYERNORM)
    assert len(variants) == 2
    # mean 1: x - mean is 0 or 2^-23, the row maximum sits on every second-half entry -> codes 0 / 127;
    # mean 1 + 2^-23: x - mean is -2^-23 or 0 -> codes -127 / 0. Same magnitude, so the same step.
    codes = sorted(tuple(q[0].tolist()) for q, _ in variants)
    assert codes == sorted([tuple([0] * 32 + [127] * 32), tuple([-127] * 32 + [0] * 32)])
    steps = {float(s[0]) for _, s in variants}
    assert len(steps) == 1 and steps.pop() > 0
    ys = O.row_y_variants(x, "f32", O.LAYERNORM)
    assert len(ys) == 2 and all(y.shape == (1, 64) for y in ys)


def _var_near_midpoint_row():
    """64 values with mean 0: +-1 (20), +-2 (42) and +-(1 + 2^-19). The exact variance is
    190/64 + 2^-23 + 2^-43: 2^-43 above the midpoint of the binary32 neighbours 2.96875 and
    2.96875 + 2^-22, i.e. 2^-21 spacings from it."""
    c = 1.0 + 2.0 ** -19
    return np.array([1.0, -1.0] * 10 + [2.0, -2.0] * 21 + [c, -c], F32)


def test_variance_next_to_a_midpoint_gives_both_roundings():
    x = _var_near_midpoint_row()
    exact = sum(Fraction(float(v)) ** 2 for v in x) / 64 - (sum(Fraction(float(v)) for v in x) / 64) ** 2
    assert exact == Fraction(190, 64) + Fraction(1, 2 ** 23) + Fraction(1, 2 ** 43)
    st = O.row_stats(x, O.LAYERNORM)
    assert st["mu"] == F32(0.0)
    assert st["var"] == F32(2.96875 + 2.0 ** -22) and st["var_other"] == F32(2.96875)
    assert st["var_dist"] == 2.0 ** -21
    ys = O.row_y_variants(x, "f32", O.LAYERNORM)
    assert len(ys) == 2
    # y = x * rstd with rstd = fl32(1 / fl32(sqrt(fl32(var + eps)))): each variance gives its own rstd,
    # and the entries equal to 1 take exactly that value
    eps = F32(1e-5)
    rstd = sorted(float(F32(1.0) / np.sqrt(F32(v) + eps)) for v in (st["var"], st["var_other"]))
    assert rstd[0] < rstd[1]
    assert sorted(float(y[0, 0]) for y in ys) == rstd
    # codes are scale-free here (every |x| is 1, 2 or c), so the two roundings share them
    variants = O.norm_quant_row_variants(x, "f32", O.LAYERNORM)
    assert len({tuple(q[0].tolist()) for q, _ in variants}) == 1


def test_rows_without_a_near_tie_give_one_variant():
    rng = np.random.default_rng(5)
    for norm in (O.LAYERNORM, O.RMSNORM, O.NONE):
        x = rng.standard_normal(256).astype(F32)
        gamma = (1 + 0.1 * rng.standard_normal(256)).astype(F32)
        variants = O.norm_quant_row_variants(x, "f32", norm, gamma)
        q, step, _ = O.norm_quant(x[None, :], "f32", norm, gamma)
        assert len(variants) == 1
        assert np.array_equal(variants[0][0], q) and variants[0][1][0] == step[0]


def test_row_variants_pin_catches_planted_mistakes(monkeypatch):
    # the far neighbour dropped: only the oracle's own rounding is offered
    def only_own(x_row, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5):
        x32 = O.widen(np.asarray(x_row)[None, :], dtype)
        st = O.row_stats(x32[0], norm)
        return [O.normalize(x32, norm, [st["mu"]], [st["var"]], gamma_f, beta_f, eps)]

    # the mean's alternative taken for the variance as well
    def crossed(x_row, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5):
        x32 = O.widen(np.asarray(x_row)[None, :], dtype)
        st = O.row_stats(x32[0], norm)
        return [O.normalize(x32, norm, [mu], [st["var"] if mu == st["mu"] else st["mu_other"]], gamma_f, beta_f,
                            eps) for mu in (st["mu"], st["mu_other"])]

    for mutant in (only_own, crossed):
        monkeypatch.setattr(OM, "row_y_variants", mutant)
        with pytest.raises(AssertionError):
            test_mean_on_a_midpoint_gives_both_roundings()
