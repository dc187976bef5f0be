"""Pins of the CPU oracle to facts fixed outside it (pages' printed values, closed forms,
textbook special cases, independent library routines, brute force). CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- rounding primitives

def test_rn32_rational_matches_binary64_to_binary32_cast():
    # numpy's float64 -> float32 cast is correctly rounded (ties to even); every float64 is a rational.
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
        rng.standard_normal(500) * 1e-42,                     # binary32 subnormal range
    ])
    for v in vals.tolist():
        f = Fraction(v)
        got, dist, other = O.rn32_rational(f.numerator, f.denominator)
        assert got == np.float32(v), v
        assert 0.0 <= dist <= 0.5
        assert got != other or v == 0.0


def test_rn32_rational_exact_midpoints_go_to_even():
    for m in [1 << 23, (1 << 23) + 1, (1 << 24) - 1, 12345677]:
        for e in [-149, -130, -20, 0, 17]:
            # midpoint between m*2^e and (m+1)*2^e
            num, den = (2 * m + 1, 1 << (1 - e)) if e < 1 else ((2 * m + 1) << (e - 1), 1)
            got, dist, other = O.rn32_rational(num, den)
            even = m if m % 2 == 0 else m + 1
            assert got == F32(math.ldexp(even, e))
            assert dist == 0.0


def test_bf16_and_f16_output_rounding_match_torch_casts():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000)).astype(F32)
    # include exact bf16 midpoints
    mids = ((rng.integers(0, 1 << 15, 1000).astype(np.uint32) << 16) | 0x8000).view(F32)
    v = np.concatenate([v, mids[np.isfinite(mids)]])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.round_output(v, "bf16"), ref)
    ref16 = torch.from_numpy(v).to(torch.float16).numpy()
    got16 = O.round_output(v, "f16")
    assert np.array_equal(got16.view(np.uint16), ref16.view(np.uint16))


def test_widen_bf16_bits():
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.widen(bits, "bf16"), x.float().numpy())


# --------------------------------------------------------------------------- statistics (R2)

def test_row_stats_closed_form_alternating_row():
    # x = c + d, c - d alternating over an even K: mean c and variance d^2 exactly.
    for c, d, k in [(0.5, 0.25, 64), (-3.0, 1.5, 4096), (100.0, 0.125, 20480), (0.0, 2.0 ** -20, 512)]:
        row = np.empty(k, F32)
        row[0::2], row[1::2] = c + d, c - d
        st = O.row_stats(row, O.LAYERNORM)
        assert st["mu"] == F32(c) and st["var"] == F32(d * d)
        rms = O.row_stats(row, O.RMSNORM)
        assert rms["var"] == F32(c * c + d * d)


def test_row_stats_agree_with_float64_within_one_ulp():
    rng = np.random.default_rng(2)
    for k in [64, 1000, 4096]:
        for _ in range(20):
            row = (rng.standard_normal(k) * 3 + rng.standard_normal()).astype(F32)
            st = O.row_stats(row, O.LAYERNORM)
            r64 = row.astype(np.float64)
            for got, ref in [(st["mu"], r64.mean()), (st["var"], r64.var())]:
                assert abs(float(got) - ref) <= np.spacing(F32(abs(ref))) * 1.01 + 1e-30
            ms = O.row_stats(row, O.RMSNORM)["var"]
            ref = np.mean(r64 * r64)
            assert abs(float(ms) - ref) <= np.spacing(F32(ref)) * 1.01


def test_layernorm_output_has_zero_mean_unit_variance():
    # Textbook LayerNorm with gamma = 1, beta = 0 (and eps -> 0): every row has mean 0, variance 1.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((16, 2048)) * 5 + 7).astype(np.float16)
    x32 = O.widen(x, "f16")
    st = [O.row_stats(r, O.LAYERNORM) for r in x32]
    y = O.normalize(x32, O.LAYERNORM, [s["mu"] for s in st], [s["var"] for s in st], eps=0.0)
    y64 = y.astype(np.float64)
    assert np.all(np.abs(y64.mean(axis=1)) < 1e-5)
    assert np.all(np.abs(y64.var(axis=1) - 1.0) < 1e-5)
    # RMSNorm: unit mean square
    st = [O.row_stats(r, O.RMSNORM) for r in x32]
    y = O.normalize(x32, O.RMSNORM, var=[s["var"] for s in st], eps=0.0).astype(np.float64)
    assert np.all(np.abs(np.mean(y * y, axis=1) - 1.0) < 1e-5)


# --------------------------------------------------------------------------- per-token quantisation (R1)

def test_quantize_round_half_to_even_ties():
    # absmax 127 -> step exactly 1.0, so v/step = v and the ties are exact.
    y = np.array([[2.5, 3.5, -2.5, 127.0, 0.5, 1.5, -0.5, -126.5]], F32)
    q, step = O.quantize_rows(y)
    assert step[0] == F32(1.0)
    assert q[0].tolist() == [2, 4, -2, 127, 0, 2, 0, -126]


def test_quantize_row_invariants():
    rng = np.random.default_rng(4)
    y = (rng.standard_normal((300, 512)) * 10.0 ** rng.integers(-8, 8, (300, 1))).astype(F32)
    y[5] = 0.0
    y[6] = -0.0
    q, step = O.quantize_rows(y)
    for i in range(y.shape[0]):
        if step[i] == 0:
            assert not q[i].any()
            continue
        assert np.max(np.abs(q[i].astype(int))) == 127
        err = np.abs(q[i].astype(np.float64) * float(step[i]) - y[i].astype(np.float64))
        assert np.all(err <= float(step[i]) / 2 * (1 + 2.0 ** -15))
    assert q.min() >= -127


def test_page3_outlier_row_example():
    g = _golden("p3_fix1_outlier_row.json")
    k, pr = g["row"]["k"], g["printed"]
    rng = np.random.default_rng(5)
    row = rng.uniform(g["row"]["ordinary_low"], g["row"]["ordinary_high"], k).astype(F32)
    row[0], row[1] = g["row"]["ordinary_high"], g["row"]["ordinary_low"]   # the stated range is reached
    for ch, v in g["row"]["outliers"].items():
        row[int(ch)] = v
    q, step, _ = O.norm_quant(row[None, :], "f32", O.NONE)
    assert step[0] == F32(60.0) / F32(127.0)
    assert abs(float(step[0]) - pr["step_with_outliers"]) < g["printed_precision"]["step_with_outliers"]
    assert q[0, 1512] == 95 and q[0, 2817] == -127
    ordinary = np.delete(q[0], [1512, 2817])
    assert len(np.unique(ordinary)) == pr["ordinary_levels"]
    assert ordinary.min() == -4 and ordinary.max() == 4
    _, step2, _ = O.norm_quant(np.delete(row, [1512, 2817])[None, :], "f32", O.NONE)
    assert abs(float(step2[0]) - pr["step_without_outliers"]) < g["printed_precision"]["step_without_outliers"]
    assert float(step[0]) / float(step2[0]) == pytest.approx(pr["finer_factor"], rel=1e-6)


# --------------------------------------------------------------------------- smoothing factors and fold (R4)

def test_smoothing_factors_exact_on_powers_of_two():
    # a = 2^p, w = 2^r: s = 2^(alpha p - (1 - alpha) r), exact when the exponent is an integer.
    for alpha in [0.0, 0.25, 0.5, 0.75, 1.0]:
        for p in range(-12, 13, 4):
            for r in range(-12, 13, 4):
                e = alpha * p - (1 - alpha) * r
                s, dist, _ = O.smoothing_factors([2.0 ** p], [2.0 ** r], alpha)
                assert s[0] == F32(max(2.0 ** e, F32(1e-5))), (alpha, p, r)


def test_smoothing_factors_match_binary64_formula():
    rng = np.random.default_rng(6)
    a = (np.abs(rng.standard_normal(2000)) * 10.0 ** rng.integers(-3, 3, 2000)).astype(F32)
    w = (np.abs(rng.standard_normal(2000)) * 10.0 ** rng.integers(-4, 1, 2000)).astype(F32)
    a, w = np.maximum(a, F32(2e-5)), np.maximum(w, F32(2e-5))      # stay clear of the eps clamps
    for alpha in [0.5, 0.8]:
        s, dist, other = O.smoothing_factors(a, w, alpha)
        ref = np.power(a.astype(np.float64), alpha) / np.power(w.astype(np.float64), 1.0 - alpha)
        assert np.all(np.abs(s.astype(np.float64) - ref) <= 0.5000001 * np.spacing(ref.astype(F32)).astype(np.float64))
        assert np.mean(s == ref.astype(F32)) > 0.999


def test_smoothing_eps_clamps():
    s, _, _ = O.smoothing_factors([0.0, 0.0, 1.0], [0.0, 1.0, 0.0], 0.5)
    eps = F32(1e-5)
    assert s[0] == F32(1.0)                                  # eps^0.5 / eps^0.5
    assert s[1] == F32(math.sqrt(float(eps)))                # clamped activation max
    assert s[2] == F32(1.0 / math.sqrt(float(eps)))          # clamped weight max


def _fixture_layer(alpha, k=256, n=192, m_cal=64, seed=7, norm=O.NONE):
    rng = np.random.default_rng(seed)
    x_cal = rng.standard_normal((m_cal, k)).astype(F32)
    x_cal[:, [3, 77, 200]] *= 50.0
    w = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    return x_cal, w


def test_equivalence_before_quantization():
    # Y = X W^T must be unchanged by the fold up to the binary32 roundings of gamma' and W-hat
    # ("LLM.int8() and SmoothQuant", going deeper; "SmoothQuant, in depth", failure modes:
    # check logits right after smoothing, before quantising).
    x_cal, w = _fixture_layer(0.5)
    a, _ = O.calibrate(x_cal, "f32", O.NONE)
    f = O.fold(a, w, "f32", 0.5)
    x = x_cal[:16].astype(np.float64)
    y_ref = x @ w.astype(np.float64).T
    y_s = (x * f["gamma_f"].astype(np.float64)) @ f["w_hat"].astype(np.float64).T
    bound = 2.0 ** -22 * (np.abs(x) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(y_s - y_ref) <= bound)
    # with the exact (binary64) 1/s and W*s the identity holds to binary64 rounding
    s64 = f["s"].astype(np.float64)
    y_e = (x / s64) @ (w.astype(np.float64) * s64).T
    assert np.max(np.abs(y_e - y_ref)) <= 1e-12 * np.max(np.abs(y_ref))


def test_equivalence_through_layernorm_fold():
    rng = np.random.default_rng(8)
    k, n = 512, 64
    x = (rng.standard_normal((8, k)) * 2).astype(np.float16)
    x[:, [10, 300]] *= 40
    gamma = (1 + 0.1 * rng.standard_normal(k)).astype(F32)
    beta = (0.1 * rng.standard_normal(k)).astype(F32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    a, info = O.calibrate(x, "f16", O.LAYERNORM, gamma, beta)
    f = O.fold(a, w, "f32", 0.5, norm=O.LAYERNORM, gamma=gamma, beta=beta)
    y_plain = info["y"].astype(np.float64) @ w.astype(np.float64).T
    _, _, qi = O.norm_quant(x, "f16", O.LAYERNORM, f["gamma_f"], f["beta_f"])
    y_fold = qi["y"].astype(np.float64) @ f["w_hat"].astype(np.float64).T
    scale = np.abs(info["y"].astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    assert np.all(np.abs(y_fold - y_plain) <= 2.0 ** -20 * scale + 1e-12)


def test_alpha_half_gives_equal_channel_maxima():
    # alpha = 0.5: both X-hat and W-hat have channel maxima sqrt(max|X_j| max|W_j|).
    x_cal, w = _fixture_layer(0.5)
    a, _ = O.calibrate(x_cal, "f32", O.NONE)
    f = O.fold(a, w, "f32", 0.5)
    xmax = np.max(np.abs(x_cal * f["gamma_f"]), axis=0).astype(np.float64)
    wmax = np.max(np.abs(f["w_hat"]), axis=0).astype(np.float64)
    geo = np.sqrt(a.astype(np.float64) * f["w_colmax"].astype(np.float64))
    assert np.all(np.abs(xmax / geo - 1) < 2.0 ** -21)
    assert np.all(np.abs(wmax / geo - 1) < 2.0 ** -21)


def test_alpha_endpoints():
    x_cal, w = _fixture_layer(0.5)
    a, _ = O.calibrate(x_cal, "f32", O.NONE)
    f1 = O.fold(a, w, "f32", 1.0)       # all of the activation range moves: smoothed act maxima = 1
    assert np.all(np.abs(np.max(np.abs(x_cal * f1["gamma_f"]), axis=0) - 1) < 2.0 ** -21)
    f0 = O.fold(a, w, "f32", 0.0)       # s = 1 / max|W_j|: smoothed weight column maxima = 1
    assert np.all(np.abs(np.max(np.abs(f0["w_hat"]), axis=0) - 1) < 2.0 ** -21)


def test_page4_two_channel_example():
    g = _golden("p4_two_channel_example.json")
    pr, tol = g["printed"], g["printed_precision"]
    act, wmax = g["act_max"], g["w_max"]
    x_cal = np.array([[act[0], -0.5], [-3.0, act[1]]], F32)
    w = np.array([[wmax[0], -0.1], [0.05, wmax[1]], [-0.2, 0.25]], F32)    # column maxima 0.2, 0.5
    a, _ = O.calibrate(x_cal, "f32", O.NONE)
    assert a.tolist() == [60.0, 1.0]
    step0 = float(np.max(a)) / 127
    assert abs(step0 - pr["before"]["step"]) < tol["step"]
    assert abs(float(a[1]) / step0 - pr["before"]["channel2_levels"]) < tol["levels"] + 0.2
    for key, alpha in [("alpha_0.5", 0.5), ("alpha_0.8", 0.8)]:
        f = O.fold(a, w, "f32", alpha)
        xs_max = (a * f["gamma_f"]).astype(np.float64)           # smoothed activation channel maxima
        _, step, _ = O.norm_quant(xs_max[None, :].astype(F32), "f32", O.NONE)
        levels2 = xs_max[1] / float(step[0])
        assert abs(levels2 - pr[key]["channel2_levels"]) < tol["levels"]
        if "step" in pr[key]:
            assert abs(float(np.max(xs_max)) - pr[key]["step_numerator"]) < tol["step_numerator"]
            assert abs(float(step[0]) - pr[key]["step"]) < tol["step"]
        if "weight_range" in pr[key]:
            wm = np.max(np.abs(f["w_hat"]), axis=0).astype(np.float64)
            assert abs(wm.max() / wm.min() - pr[key]["weight_range"]) < tol["weight_range"]


def test_shared_s_over_concatenated_projections():
    # q/k/v share one s from the elementwise max of their weight maxima; per-output-channel
    # quantisation is per row, so folding the concatenation equals folding each part with that s.
    rng = np.random.default_rng(9)
    k = 128
    parts = [(rng.standard_normal((n, k)) * sc).astype(F32) for n, sc in [(32, 0.02), (48, 0.05), (16, 0.01)]]
    a = (np.abs(rng.standard_normal(k)) * 5).astype(F32)
    cat = O.fold(a, np.concatenate(parts), "f32", 0.8)
    wmax = np.max(np.stack([O.weight_colmax(p, "f32") for p in parts]), axis=0)
    assert np.array_equal(cat["w_colmax"], wmax)
    row0 = 0
    for p in parts:
        f = O.fold(a, p, "f32", 0.8, s=cat["s"])
        assert np.array_equal(f["wq"], cat["wq"][row0:row0 + len(p)])
        assert np.array_equal(f["w_scale"], cat["w_scale"][row0:row0 + len(p)])
        row0 += len(p)


def test_calibration_is_a_running_max():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((40, 256)) * 3).astype(np.float16)
    g = (1 + 0.1 * rng.standard_normal(256)).astype(F32)
    b = (0.1 * rng.standard_normal(256)).astype(F32)
    full, _ = O.calibrate(x, "f16", O.LAYERNORM, g, b)
    a1, _ = O.calibrate(x[:17], "f16", O.LAYERNORM, g, b)
    a2, _ = O.calibrate(x[17:], "f16", O.LAYERNORM, g, b, absmax=a1)
    assert np.array_equal(full, a2)
    none, _ = O.calibrate(x, "f16", O.NONE)
    assert np.array_equal(none, np.max(np.abs(x.astype(F32)), axis=0))


# --------------------------------------------------------------------------- GEMM and epilogue (R6)

def test_int_gemm_equals_brute_force():
    rng = np.random.default_rng(11)
    for m, n, k in [(1, 1, 64), (3, 5, 64), (17, 9, 128), (16, 40, 192), (40, 16, 256)]:
        xq = rng.integers(-127, 128, (m, k), dtype=np.int64).astype(np.int8)
        wq = rng.integers(-127, 128, (n, k), dtype=np.int64).astype(np.int8)
        assert np.array_equal(O.int_gemm(xq, wq), O.int_gemm_loops(xq, wq))


def test_int_gemm_extreme_k_stays_exact():
    k = 133120                                         # largest K whose |acc| <= K * 127^2 fits int32
    xq = np.full((2, k), 127, np.int8)
    xq[1] = -127
    wq = np.full((1, k), 127, np.int8)
    acc = O.int_gemm(xq, wq)
    assert acc[0, 0] == k * 127 * 127 == 2147092480 and acc[1, 0] == -2147092480
    assert acc[0, 0] < 2 ** 31


def test_dequantize_rounding():
    acc = np.array([[2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 24 + 1), 7]], np.int64)
    out, v = O.dequantize(acc, np.array([1.0], F32), np.array([1.0, 1.0, 1.0, 0.5], F32))
    assert v[0].tolist() == [2.0 ** 24, 2.0 ** 24 + 4, -(2.0 ** 24), 3.5]
    out16, _ = O.dequantize(np.array([[2049]]), np.array([1.0], F32), np.array([1.0], F32), out_dtype="f16")
    assert float(out16[0, 0]) == 2048.0                  # 2049 lies halfway: ties to even in fp16
    # powers of two scales make every step exact: compare with binary64 directly
    rng = np.random.default_rng(12)
    acc = rng.integers(-2 ** 20, 2 ** 20, (8, 8))
    xs = (2.0 ** rng.integers(-10, 0, 8)).astype(F32)
    ws = (2.0 ** rng.integers(-10, 0, 8)).astype(F32)
    _, v = O.dequantize(acc, xs, ws)
    assert np.array_equal(v.astype(np.float64), acc * xs[:, None].astype(np.float64) * ws[None, :].astype(np.float64))


def test_whole_layer_close_to_float_product():
    # W8A8 with smoothing stays close to the unquantised product on outlier-heavy inputs
    # (the point of the method), and much closer than without smoothing.
    rng = np.random.default_rng(13)
    k, n = 512, 256
    x_cal = rng.standard_normal((64, k)).astype(F32)
    x = rng.standard_normal((16, k)).astype(F32)
    cols = [5, 50, 100, 400]
    x_cal[:, cols] *= 50
    x[:, cols] *= 50
    w = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    r = O.w8a8_linear(x, x_cal, w, "f32", O.NONE, 0.5)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    err_s = np.linalg.norm(r["out32"] - ref) / np.linalg.norm(ref)
    xq, xs = O.quantize_rows(x)
    wq, ws = O.quantize_rows(w)
    _, plain = O.dequantize(O.int_gemm(xq, wq), xs, ws)
    err_p = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    assert err_s < 0.02 and err_s < 0.5 * err_p
