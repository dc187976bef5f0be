"""Pins of the oracle's per-tensor FP8 functions (reading R18) to facts fixed outside them: E4M3 codes
worked by hand from the format's definition, saturation at the largest finite value, the reduction to
the pinned per-row FP8 quantiser, nearest-value brute force, and the static step's definition. CPU only."""
import numpy as np
import pytest

import oracle as O

F32 = np.float32
GRID = np.sort(np.unique(np.abs(O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64))))


def test_quantize_tensor_fp8_hand_worked_and_saturating():
    # step 1: codes are the E4M3 values themselves; 0.3 -> 1.25 * 2^-2 (0x2A); beyond 448 saturates
    y = np.array([[1.0, 0.3, -2.0, 448.0], [464.0, 465.0, 500.0, -1000.0]], F32)
    q, step = O.quantize_tensor_fp8(y, 1.0)
    assert step == F32(1.0)
    assert q.tolist() == [[0x38, 0x2A, 0xC0, 0x7E], [0x7E, 0x7E, 0x7E, 0xFE]]
    assert not np.isin(q, [0x7F, 0xFF]).any()                                  # never NaN
    # the same values through the per-row quantiser of the format alone give NaN past the 464 midpoint
    assert O.e4m3_encode(np.array([465.0], F32))[0] == 0x7F


def test_dynamic_step_maps_the_tensor_max_to_448():
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((7, 50)) * 30).astype(F32)
    y[4, 17] = -150.0                                                            # the tensor max
    q, step = O.quantize_tensor_fp8(y)
    assert step == F32(np.max(np.abs(y))) / F32(448)
    assert q[4, 17] == 0xFE and np.abs(O.e4m3_decode(q)).max() == 448.0


def test_one_row_reduces_to_the_per_row_quantiser():
    rng = np.random.default_rng(4)
    for _ in range(20):
        y = (rng.standard_normal((1, 64)) * np.exp(rng.uniform(-8, 8))).astype(F32)
        q, step = O.quantize_tensor_fp8(y)
        q1, s1 = O.quantize_rows_fp8(y)
        assert np.array_equal(q, q1) and step == s1[0]


@pytest.mark.parametrize("step", [0.0, -1.0])
def test_non_positive_step_gives_zero_codes(step):
    q, st = O.quantize_tensor_fp8(np.array([[1.0, -3.0]], F32), step)
    assert not q.any()


def test_codes_are_the_nearest_e4m3_value_of_the_clipped_quotient():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((6, 40)) * 40).astype(F32)
    for step in [F32(0.05), F32(0.3), F32(1.7)]:                                   # the first clips many values
        q, _ = O.quantize_tensor_fp8(y, step)
        t = np.clip((y / step).astype(F32).astype(np.float64), -448.0, 448.0)
        dec = O.e4m3_decode(q).astype(np.float64)
        for tv, d, c in zip(t.ravel(), dec.ravel(), q.ravel()):
            i = np.searchsorted(GRID, abs(tv))
            cands = GRID[max(0, i - 1):i + 1]
            best = np.min(np.abs(cands - abs(tv)))
            assert abs(abs(d) - abs(tv)) == best
            assert d == 0 or np.sign(d) == np.sign(tv)
            if np.count_nonzero(np.abs(cands - abs(tv)) == best) == 2:
                assert (int(c) & 1) == 0                                        # ties to the even mantissa


def test_static_step_fp8_hand_worked():
    # max_j a_j / s_j = max(10 / 1, 448 / 2, 3 / 0.5) = 224 -> step 224 / 448 = 0.5
    assert O.static_step_fp8(np.array([10.0, 448.0, 3.0], F32), np.array([1.0, 2.0, 0.5], F32)) == F32(0.5)
    # the division comes before the max: a larger a_j can lose to a smaller one with a smaller s_j
    assert O.static_step_fp8(np.array([100.0, 8.0], F32), np.array([10.0, 0.5], F32)) == F32(16.0) / F32(448)


def test_fold_fp8_per_tensor_step_is_the_largest_row_step():
    rng = np.random.default_rng(6)
    a = (np.abs(rng.standard_normal(64)) * 5 + 0.1).astype(F32)
    w = (rng.standard_normal((9, 64)) * 0.02).astype(F32)
    f = O.fold_fp8_per_tensor(a, w, "f32", 0.5)
    per_row = O.fold_fp8(a, w, "f32", 0.5)
    assert np.all(f["w_scale"] == np.max(per_row["w_scale"]))
    q, st = O.quantize_tensor_fp8(f["w_hat"], f["w_scale"][0])
    assert np.array_equal(q, f["wq"])


def test_norm_quant_fp8_per_tensor_is_the_norm_then_the_tensor_quantiser():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 64)).astype(F32)
    g = (1 + 0.1 * rng.standard_normal(64)).astype(F32)
    b = (0.1 * rng.standard_normal(64)).astype(F32)
    for step in [None, F32(0.004)]:
        q, xs, info = O.norm_quant_fp8_per_tensor(x, "f32", "layernorm", g, b, 1e-5, step)
        q2, s2 = O.quantize_tensor_fp8(info["y"], step)
        assert np.array_equal(q, q2) and np.all(xs == s2)


def test_the_tensor_max_sets_every_row_step():
    # doubling the row that holds the tensor max doubles the one step, so every other row's codes
    # shrink; with a step per row they would not move
    rng = np.random.default_rng(8)
    y = (rng.standard_normal((6, 48)) * 20).astype(F32)
    y[2, 5] = 150.0
    q1, s1 = O.quantize_tensor_fp8(y)
    y2 = y.copy()
    y2[2] *= F32(2)
    q2, s2 = O.quantize_tensor_fp8(y2)
    assert s2 == F32(2) * s1
    d1, d2 = np.abs(O.e4m3_decode(q1)), np.abs(O.e4m3_decode(q2))
    others = np.arange(6) != 2
    assert np.all(d2[others].max(axis=1) < d1[others].max(axis=1))
    assert d1[2].max() == d2[2].max() == 448.0
