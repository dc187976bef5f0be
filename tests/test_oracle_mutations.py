"""Planted mistakes in the oracle (on the CPU only): each plausible slip must trip a pin.

Every case patches one oracle function with a wrong variant, re-runs the pin
that should catch it, and expects that pin to fail.
"""
import numpy as np
import pytest

import oracle
import oracle.smoothquant_oracle as OM
import tests.test_oracle_pins as P

F32 = np.float32


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(OM, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(pin):
    with pytest.raises((AssertionError, ValueError)):
        pin()


def test_step_over_128_is_caught(monkeypatch):
    good = OM.quantize_rows

    def bad(y):
        y = np.atleast_2d(np.asarray(y, F32))
        step = (np.max(np.abs(y), axis=1) / F32(128)).astype(F32)
        q = np.clip(np.rint(y / step[:, None]), -127, 127)
        return q.astype(np.int8), step
    _patch(monkeypatch, "quantize_rows", bad)
    _fails(P.test_page3_outlier_row_example)
    _patch(monkeypatch, "quantize_rows", good)
    P.test_page3_outlier_row_example()


def test_round_half_away_from_zero_is_caught(monkeypatch):
    def bad(y):
        y = np.atleast_2d(np.asarray(y, F32))
        step = (np.max(np.abs(y), axis=1) / F32(127)).astype(F32)
        t = y / step[:, None]
        q = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127)
        return q.astype(np.int8), step
    _patch(monkeypatch, "quantize_rows", bad)
    _fails(P.test_quantize_round_half_to_even_ties)


def test_wrong_weight_exponent_is_caught(monkeypatch):
    def bad(act_absmax, w_colmax, alpha, eps=1e-5):      # w^alpha instead of w^(1 - alpha)
        a1 = np.maximum(np.asarray(act_absmax, F32), F32(eps)).astype(np.float64)
        w1 = np.maximum(np.asarray(w_colmax, F32), F32(eps)).astype(np.float64)
        s = np.maximum((a1 ** alpha / w1 ** alpha).astype(F32), F32(eps))
        return s, np.full(s.size, 0.5), s
    _patch(monkeypatch, "smoothing_factors", bad)
    _fails(P.test_alpha_endpoints)


def test_inverted_migration_direction_is_caught(monkeypatch):
    good = OM.smoothing_factors

    def bad(act_absmax, w_colmax, alpha, eps=1e-5):      # activations multiplied, weights divided
        s, d, o = good(act_absmax, w_colmax, alpha, eps)
        return (F32(1) / s).astype(F32), d, o
    _patch(monkeypatch, "smoothing_factors", bad)
    _fails(P.test_alpha_half_gives_equal_channel_maxima)
    _fails(P.test_page4_two_channel_example)


def test_fold_on_output_rows_is_caught(monkeypatch):
    good = OM.fold

    def bad(act_absmax, w, dtype, alpha, eps=1e-5, norm="none", gamma=None, beta=None, s=None):
        w32 = OM.widen(w, dtype)
        r = good(act_absmax, w, dtype, alpha, eps, norm, gamma, beta, s)
        sq = min(w32.shape)                               # scales rows instead of columns
        w_hat = w32.copy()
        w_hat[:sq] = w32[:sq] * r["s"][:sq, None]
        r["w_hat"] = w_hat
        return r
    _patch(monkeypatch, "fold", bad)
    _fails(P.test_equivalence_before_quantization)


def test_uncentred_layernorm_variance_is_caught(monkeypatch):
    good = OM.row_stats

    def bad(x32_row, norm):
        st = good(x32_row, norm)
        if norm == OM.LAYERNORM:
            st["var"] = F32(np.mean(x32_row.astype(np.float64) ** 2))
        return st
    _patch(monkeypatch, "row_stats", bad)
    _fails(P.test_row_stats_closed_form_alternating_row)


def test_transposed_scales_in_epilogue_are_caught(monkeypatch):
    def bad(acc, x_scale, w_scale, bias=None, out_dtype="f32"):
        v = np.asarray(acc).astype(F32) * np.asarray(x_scale, F32)[None, :]
        v = v * np.asarray(w_scale, F32)[:, None]
        return OM.round_output(v, out_dtype), v
    _patch(monkeypatch, "dequantize", bad)
    _fails(P.test_dequantize_rounding)


def test_transposed_gemm_operand_is_caught(monkeypatch):
    def bad(xq, wq, block=512):
        return (np.asarray(xq).astype(np.float64).T @ np.asarray(wq).astype(np.float64)).astype(np.int64)
    _patch(monkeypatch, "int_gemm", bad)
    _fails(P.test_int_gemm_equals_brute_force)
