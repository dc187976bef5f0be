"""Pins of the oracle's per-tensor granularities (one INT8 step for a whole tensor, dynamic
or static calibrated; per-tensor weights) to facts fixed outside those functions: hand-worked
values, clipping and zero cases, exact rational brute force, the single-row special case that
reduces to the pinned per-row quantiser, and invariants. CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

F32 = np.float32


def _rne_int(fr: Fraction) -> int:
    """Round a rational half to even."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def test_quantize_tensor_hand_worked():
    # amax 254 -> step 2 exactly; 127 / 2 = 63.5 -> 64 (even), 1 / 2 = 0.5 -> 0 (even), -254 / 2 = -127
    y = np.array([[-254.0, 0.5], [1.0, 127.0]], F32)
    q, st = O.quantize_tensor(y)
    assert st == F32(2.0)
    assert q.tolist() == [[-127, 0], [0, 64]]


def test_quantize_tensor_static_clips():
    # step 1: values past +-127.5 clip; 126.5 -> 126 (even); 127.5 -> 128 -> clipped to 127; -0.5 -> 0
    y = np.array([[300.0, -300.0, 126.5, 127.5, -0.5, -127.5]], F32)
    q, st = O.quantize_tensor(y, step=1.0)
    assert st == F32(1.0)
    assert q.tolist() == [[127, -127, 126, 127, 0, -127]]


def test_quantize_tensor_zero_and_nonpositive_steps():
    q, st = O.quantize_tensor(np.zeros((3, 5), F32))
    assert st == 0 and not q.any()
    q, _ = O.quantize_tensor(np.ones((2, 2), F32), step=0.0)
    assert not q.any()
    q, _ = O.quantize_tensor(np.ones((2, 2), F32), step=-1.0)
    assert not q.any()


def test_quantize_tensor_brute_force_rationals():
    # code = RNE(fl32(y / step)) clipped, evaluated with exact rationals on tiny tensors
    rng = np.random.default_rng(7)
    for trial in range(40):
        y = (rng.standard_normal((3, 7)) * 10.0 ** rng.integers(-3, 4)).astype(F32)
        static = trial % 2 == 1
        step = F32(np.max(np.abs(y)) / F32(127) * F32(0.6)) if static else None
        q, st = O.quantize_tensor(y, step)
        amax = max(abs(Fraction(float(v))) for v in y.ravel())
        want_step = O.rn32_rational((amax / 127).numerator, (amax / 127).denominator)[0] if not static else step
        assert st == F32(want_step)
        for v, c in zip(y.ravel().tolist(), q.ravel().tolist()):
            quo = Fraction(v) / Fraction(float(st))
            r = Fraction(float(O.rn32_rational(quo.numerator, quo.denominator)[0])) if quo != 0 else Fraction(0)
            assert c == max(-127, min(127, _rne_int(r))), (trial, v, c)


def test_single_row_tensor_equals_per_row_quantiser():
    rng = np.random.default_rng(3)
    for k in (1, 8, 1000):
        y = (rng.standard_normal((1, k)) * 5).astype(F32)
        q1, st1 = O.quantize_tensor(y)
        q2, st2 = O.quantize_rows(y)
        assert st1 == st2[0] and np.array_equal(q1, q2)


@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
def test_norm_quant_per_tensor_single_row_is_per_token(norm):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 256)).astype(F32) * 3
    g = (1 + 0.1 * rng.standard_normal(256)).astype(F32)
    b = (0.1 * rng.standard_normal(256)).astype(F32) if norm == "layernorm" else None
    q1, xs1, _ = O.norm_quant_per_tensor(x, "f32", norm, g, b)
    q2, xs2, _ = O.norm_quant(x, "f32", norm, g, b)
    assert np.array_equal(q1, q2) and np.array_equal(xs1, xs2)


def test_per_tensor_invariants_and_static_consistency():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 512)).astype(F32)
    x[:, 7] *= 60.0
    g = (1 + 0.1 * rng.standard_normal(512)).astype(F32)
    q, xs, info = O.norm_quant_per_tensor(x, "f32", "rmsnorm", g)
    st = xs[0]
    assert (xs == st).all()
    assert int(np.abs(q.astype(np.int32)).max()) == 127                      # the tensor maximum maps to 127
    y = info["y"].astype(np.float64)
    assert np.all(np.abs(q * np.float64(st) - y) <= np.float64(st) / 2 * (1 + 2.0 ** -15))
    flat = np.argsort(y.ravel(), kind="stable")                              # codes are monotone in y
    assert np.all(np.diff(q.ravel()[flat].astype(np.int32)) >= 0)
    qs, xss, _ = O.norm_quant_per_tensor(x, "f32", "rmsnorm", g, step=float(st))   # static with that step
    assert np.array_equal(qs, q) and (xss == st).all()
    qh, _, _ = O.norm_quant_per_tensor(x, "f32", "rmsnorm", g, step=float(st) / 2)  # half the step: clipping
    assert int(np.abs(qh.astype(np.int32)).max()) == 127
    assert (np.abs(qh.astype(np.int32)) >= np.minimum(2 * np.abs(q.astype(np.int32)) - 1, 127)).all()


def test_static_step_hand_worked():
    # ratios a/s = 254, 2, 6 -> step = 254 / 127 = 2 exactly
    assert O.static_step(np.array([254.0, 8.0, 3.0], F32), np.array([1.0, 4.0, 0.5], F32)) == F32(2.0)
    # ratios fl32(1/3), 127 -> step 1
    assert O.static_step(np.array([1.0, 127.0], F32), np.array([3.0, 1.0], F32)) == F32(1.0)
    # the max is taken after the division, not over a and s separately
    assert O.static_step(np.array([127.0, 100.0], F32), np.array([2.0, 0.5], F32)) == F32(200.0) / F32(127.0)


def test_fold_per_tensor():
    rng = np.random.default_rng(9)
    k, n = 64, 12
    a = np.abs(rng.standard_normal(k)).astype(F32) * 3
    w = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    f1 = O.fold_per_tensor(a, w, "f32", 0.5)
    f0 = O.fold(a, w, "f32", 0.5)
    assert np.array_equal(f1["s"], f0["s"]) and np.array_equal(f1["gamma_f"], f0["gamma_f"])
    assert (f1["w_scale"] == f1["w_scale"][0]).all()
    assert f1["w_scale"][0] == np.max(f0["w_scale"])                        # the largest per-row step
    assert int(np.abs(f1["wq"].astype(np.int32)).max()) == 127
    one = O.fold_per_tensor(a, w[:1], "f32", 0.5, s=f0["s"])                  # one output row: per-channel
    assert np.array_equal(one["wq"], f0["wq"][:1]) and one["w_scale"][0] == f0["w_scale"][0]
