"""Planted mistakes in the oracle's FP8 (OCP E4M3) and per-tensor functions (on the CPU only): each
plausible slip must trip a pin of the format's definition, a hand-worked value or an invariant.

Every case patches one oracle function with a wrong variant, re-runs the pin that should catch it,
and expects that pin to fail; the last line of each case checks that the pin passes again once the
right function is back.
"""
import numpy as np
import pytest

import oracle
import oracle.smoothquant_oracle as OM
import tests.test_oracle_fp8 as P8
import tests.test_oracle_fp8_granularity as P8T
import tests.test_oracle_granularity as PT

F32 = np.float32


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(OM, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(pin, *args):
    with pytest.raises((AssertionError, ValueError)):
        pin(*args)


def _encoder(bias=7, sub_lsb=2.0 ** -9, saturate=False, mant_round=np.rint):
    """An E4M3 encoder with one knob turned away from the format's definition."""
    def enc(v):
        v = np.asarray(v, dtype=F32)
        a = np.abs(v).astype(np.float64)
        sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
        sub = a < 2.0 ** -6
        q_sub = mant_round(a / sub_lsb).astype(np.int64)
        frac, exp = np.frexp(np.where(sub, 1.0, a))
        e = exp.astype(np.int64) - 1
        mant = mant_round((frac * 2.0 - 1.0) * 8.0).astype(np.int64)
        e = np.where(mant == 8, e + 1, e)
        mant = np.where(mant == 8, 0, mant)
        q = np.where(sub, q_sub, (e + bias) * 8 + mant)
        q = np.where(q > 0x7E, 0x7E if saturate else 0x7F, q)
        return (np.clip(q, 0, 0x7F) | sign).astype(np.uint8)
    return enc


def test_e4m3_encoder_is_itself_the_definition():
    # the helper with every knob at the format's value agrees with the oracle on every finite code
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = OM.e4m3_decode(codes)
    assert np.array_equal(_encoder()(vals), OM.e4m3_encode(vals))


def test_exponent_bias_8_is_caught(monkeypatch):
    _patch(monkeypatch, "e4m3_encode", _encoder(bias=8))
    _fails(P8.test_e4m3_hand_encoded_values)


def test_subnormal_spacing_2_pow_minus_10_is_caught(monkeypatch):
    _patch(monkeypatch, "e4m3_encode", _encoder(sub_lsb=2.0 ** -10))
    _fails(P8.test_e4m3_hand_encoded_values)


def test_saturating_encoder_is_caught(monkeypatch):
    # the per-row quantiser's encoder gives NaN past 464; only the per-tensor path clips first
    _patch(monkeypatch, "e4m3_encode", _encoder(saturate=True))
    _fails(P8.test_e4m3_hand_encoded_values)


def test_midpoints_away_from_zero_are_caught(monkeypatch):
    _patch(monkeypatch, "e4m3_encode", _encoder(mant_round=lambda t: np.floor(t + 0.5)))
    _fails(P8.test_every_code_round_trips_and_midpoints_go_to_even)


def test_truncating_encoder_is_caught(monkeypatch):
    _patch(monkeypatch, "e4m3_encode", _encoder(mant_round=np.floor))
    _fails(P8.test_e4m3_matches_torch_cast)


def test_fp8_step_over_127_is_caught(monkeypatch):
    good = OM.quantize_rows_fp8

    def bad(y):
        y = np.atleast_2d(np.asarray(y, dtype=F32))
        step = (np.max(np.abs(y), axis=1) / F32(127)).astype(F32)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = (y / step[:, None]).astype(F32)
        t[step == 0] = 0
        return OM.e4m3_encode(t), step
    _patch(monkeypatch, "quantize_rows_fp8", bad)
    _fails(P8.test_quantize_rows_fp8_invariants)
    _patch(monkeypatch, "quantize_rows_fp8", good)
    P8.test_quantize_rows_fp8_invariants()


def test_per_tensor_fp8_without_saturation_is_caught(monkeypatch):
    def bad(y, step=None):
        y = np.atleast_2d(np.asarray(y, dtype=F32))
        if step is None:
            step = F32(np.max(np.abs(y))) / F32(448)
        step = F32(step)
        if not step > 0:
            return np.zeros(y.shape, np.uint8), step
        return OM.e4m3_encode((y / step).astype(F32)), step
    _patch(monkeypatch, "quantize_tensor_fp8", bad)
    _fails(P8T.test_quantize_tensor_fp8_hand_worked_and_saturating)


def test_per_row_steps_in_the_per_tensor_fp8_quantiser_are_caught(monkeypatch):
    good = OM.quantize_tensor_fp8

    def bad(y, step=None):
        if step is not None:
            return good(y, step)
        q, steps = OM.quantize_rows_fp8(y)
        return q, F32(np.max(steps))
    _patch(monkeypatch, "quantize_tensor_fp8", bad)
    _fails(P8T.test_the_tensor_max_sets_every_row_step)
    _patch(monkeypatch, "quantize_tensor_fp8", good)
    P8T.test_the_tensor_max_sets_every_row_step()


def test_static_fp8_step_max_before_division_is_caught(monkeypatch):
    def bad(act_absmax, s):
        return F32(np.max(np.asarray(act_absmax, F32)) / np.max(np.asarray(s, F32))) / F32(448)
    _patch(monkeypatch, "static_step_fp8", bad)
    _fails(P8T.test_static_step_fp8_hand_worked)


def test_fp8_gemm_dropping_the_last_k_term_is_caught(monkeypatch):
    good = OM.gemm_fp8

    def bad(xq, wq, block=512):
        return good(np.asarray(xq)[:, :-1], np.asarray(wq)[:, :-1], block)
    _patch(monkeypatch, "gemm_fp8", bad)
    _fails(P8.test_gemm_fp8_exact_and_bound)


def test_static_int8_codes_without_clip_are_caught(monkeypatch):
    def bad(y, step=None):
        y = np.atleast_2d(np.asarray(y, dtype=F32))
        if step is None:
            step = F32(np.max(np.abs(y))) / F32(127)
        step = F32(step)
        if not step > 0:
            return np.zeros(y.shape, np.int8), step
        return np.rint(y / step).astype(np.int64).astype(np.int8), step     # wraps instead of clipping
    _patch(monkeypatch, "quantize_tensor", bad)
    _fails(PT.test_quantize_tensor_static_clips)


def test_per_tensor_int8_half_away_from_zero_is_caught(monkeypatch):
    def bad(y, step=None):
        y = np.atleast_2d(np.asarray(y, dtype=F32))
        if step is None:
            step = F32(np.max(np.abs(y))) / F32(127)
        step = F32(step)
        if not step > 0:
            return np.zeros(y.shape, np.int8), step
        t = (y / step).astype(np.float64)
        return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int8), step
    _patch(monkeypatch, "quantize_tensor", bad)
    _fails(PT.test_quantize_tensor_hand_worked)


def test_static_int8_step_max_before_division_is_caught(monkeypatch):
    def bad(act_absmax, s):
        return F32(np.max(np.asarray(act_absmax, F32)) / np.max(np.asarray(s, F32))) / F32(127)
    _patch(monkeypatch, "static_step", bad)
    _fails(PT.test_static_step_hand_worked)


def test_per_tensor_fold_with_the_smallest_row_step_is_caught(monkeypatch):
    good = OM.fold_per_tensor

    def bad(act_absmax, w, dtype, alpha, eps=OM.EPS_FOLD, norm=OM.NONE, gamma=None, beta=None, s=None):
        f = OM.fold(act_absmax, w, dtype, alpha, eps, norm, gamma, beta, s)
        st = F32(np.min(f["w_scale"]))
        f["wq"], _ = OM.quantize_tensor(f["w_hat"], st)
        f["w_scale"] = np.full(f["w_hat"].shape[0], st, F32)
        return f
    _patch(monkeypatch, "fold_per_tensor", bad)
    _fails(PT.test_fold_per_tensor)
    _patch(monkeypatch, "fold_per_tensor", good)
    PT.test_fold_per_tensor()
