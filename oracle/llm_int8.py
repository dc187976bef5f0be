"""Plain CPU oracle of the LLM.int8() mixed-precision decomposition.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's checks,
never by the product path; it shares no code with the HIP library.

What it follows ("LLM.int8() and SmoothQuant", section "Fix 1: give the
outliers their own lane (LLM.int8())" and its example "one token through a
layer", and "going deeper / LLM.int8() decomposition"): with X the linear's
input (tokens x channels) and W its weight, the outlier channels are
O = {j : max_t |X_tj| >= tau}, tau = 6. Those channels (and the matching
weights) are multiplied in 16-bit; every other channel goes through INT8 with
one absmax step per token row of X and one per output channel of W; the two
products are added. "SmoothQuant, in depth", "The problem SmoothQuant solves",
names the cost: a gather, a second GEMM and a merge.

Readings where the pages leave a step open:

R19 X is the binary32 input the linear sees: the norm applied with the model's
    own gamma, beta (no smoothing: LLM.int8() folds nothing), or x itself
    without a norm. Statistics as R2, elementwise steps as R3.
R20 O is found on the tokens of the current call (the threshold applies to the
    activations at run time), with >= as the page's set definition writes it.
R21 The 16-bit format is that of the weights when they are stored in 16 bits
    (fp16 or bf16), else fp16. X on O and W on O are rounded to it (half to
    even); their products are exact in binary32 and are summed in binary32.
    The order of that sum is not fixed, so the oracle keeps the exact sum and
    the checks allow a bounded difference (gemm16_bound).
R22 The INT8 part: each token's step is fl32(max over the channels outside O
    of |y| / 127) with R1's codes (the example's 4,094 remaining channels get
    a step of 2/127), and the codes of the channels in O are 0. The weights
    are quantised once, offline, with one step per output channel over all
    input channels (R1; the weights "can be quantised carefully once,
    offline", "The problem: activations, not weights"); the INT8 product then
    uses only the rows outside O because the activation codes on O are 0.
R23 The result is fl32(deq + acc16) (plus an optional bias fl32(. + b[n])),
    then round-half-even to the output type; deq is R6's epilogue of the INT8
    accumulator and acc16 the binary32 sum of the 16-bit products.
"""
from __future__ import annotations

import numpy as np

from .smoothquant_oracle import (LAYERNORM, NONE, RMSNORM, dequantize, f32_to_bf16_bits, int_gemm, normalize,
                                 quantize_rows, row_stats, widen)

__all__ = ["TAU", "outlier_channels", "half_format", "round16", "weights", "activations", "gemm16",
           "gemm16_bound", "decompose", "output_bound"]

F32 = np.float32
F64 = np.float64
TAU = 6.0


def outlier_channels(y, tau: float = TAU) -> np.ndarray:
    """O = {j : max_t |y_tj| >= tau}, ascending (reading R20)."""
    y = np.atleast_2d(np.asarray(y, F32))
    if y.shape[0] == 0:
        return np.zeros(0, np.int64)
    return np.where(np.max(np.abs(y), axis=0) >= F32(tau))[0].astype(np.int64)


def half_format(w_dtype: str) -> str:
    """The 16-bit format of the outlier product (reading R21)."""
    return "bf16" if w_dtype == "bf16" else "f16"


def round16(v32, fmt: str) -> np.ndarray:
    """binary32 values rounded half to even to fp16 or bf16, returned as (exact) binary32 values."""
    v32 = np.asarray(v32, F32)
    if fmt == "f16":
        return v32.astype(np.float16).astype(F32)
    return widen(f32_to_bf16_bits(v32), "bf16")


def weights(w, dtype: str):
    """Offline INT8 of W [N, K]: one step per output channel over all K (reading R22)."""
    return quantize_rows(widen(w, dtype))


def activations(x, dtype: str, norm: str, gamma=None, beta=None, eps=1e-5):
    """y, the binary32 input of the linear (reading R19): the norm with the model's own gamma, beta.

    Returns (y [M, K], near_tie [M]) with the rows whose statistics are near-ties flagged as in
    norm_quant.
    """
    x32 = widen(x, dtype)
    if norm == NONE:
        return x32.copy(), np.zeros(x32.shape[0], bool)
    if norm not in (LAYERNORM, RMSNORM):
        raise ValueError(norm)
    from .smoothquant_oracle import NEAR_TIE
    m = x32.shape[0]
    mu, var, tie = np.zeros(m, F32), np.zeros(m, F32), np.zeros(m, bool)
    for i in range(m):
        st = row_stats(x32[i], norm)
        mu[i], var[i] = st["mu"], st["var"]
        tie[i] = min(st["mu_dist"], st["var_dist"]) < NEAR_TIE
    return normalize(x32, norm, mu, var, gamma, beta, eps), tie


def gemm16(xo, wo) -> np.ndarray:
    """sum_i xo[m, i] * wo[n, i] of 16-bit values (given as binary32), in binary64.

    Each product of two fp16 or bf16 values is exact in binary64; the binary64 sum of the |O|
    products differs from the exact sum by at most |O| 2^-53 sum |products|, far inside
    gemm16_bound.
    """
    return np.asarray(xo, F64) @ np.asarray(wo, F64).T


def gemm16_bound(n_terms: int, sum_abs, k_step: int = 32) -> np.ndarray:
    """Bound on |acc16_gpu - acc16| for any binary32 summation of n_terms exact products taken
    k_step at a time (a tree of depth log2(k_step) inside each step, one accumulation per step),
    doubled so that a unit truncating instead of rounding is covered too."""
    steps = -(-max(n_terms, 1) // k_step)
    depth = int(np.log2(k_step)) + 1
    return 2.0 * (steps + depth) * 2.0 ** -24 * np.asarray(sum_abs, F64)


def decompose(x, dtype, norm, w, gamma=None, beta=None, eps=1e-5, tau=TAU, w_dtype=None, wq=None, w_scale=None,
              bias=None, out_dtype="f32", outliers=None):
    """The whole decomposition of one linear: Y = X_O W_O (16-bit) + dequantised INT8 product of the rest.

    x [M, K] in dtype, w [N, K] in w_dtype (default dtype); wq / w_scale default to weights(w).
    `outliers` (ascending channel indices) replaces O found on these rows: to continue from the set
    a whole batch gave when x holds only some of its rows.
    Returns a dict: y (the linear's input), near_tie, O, xq / x_scale (INT8 part, codes 0 on O),
    wq / w_scale, acc (int64), deq (binary32, before any bias), xo [M, |O|] and wo [N, |O|] (16-bit
    values), acc16 (binary64), sum_abs16 (sum of |products|), ref (binary64 deq + acc16 + bias).
    """
    w_dtype = w_dtype or dtype
    y, tie = activations(x, dtype, norm, gamma, beta, eps)
    outl = outlier_channels(y, tau) if outliers is None else np.asarray(outliers, np.int64)
    y_int = y.copy()
    y_int[:, outl] = F32(0.0)
    xq, xs = quantize_rows(y_int)
    if wq is None:
        wq, w_scale = weights(w, w_dtype)
    acc = int_gemm(xq, wq)
    _, deq = dequantize(acc, xs, w_scale)
    fmt = half_format(w_dtype)
    xo = round16(y[:, outl], fmt)
    wo = round16(widen(w, w_dtype)[:, outl], fmt)
    acc16 = gemm16(xo, wo)
    sum_abs = gemm16(np.abs(xo), np.abs(wo))
    ref = deq.astype(F64) + acc16
    if bias is not None:
        ref = ref + np.asarray(bias, F64)[None, :]
    return {"y": y, "near_tie": tie, "O": outl, "xq": xq, "x_scale": xs, "wq": wq, "w_scale": w_scale,
            "acc": acc, "deq": deq, "xo": xo, "wo": wo, "acc16": acc16, "sum_abs16": sum_abs, "ref": ref,
            "fmt": fmt, "out_dtype": out_dtype}


def output_bound(d, n_pad=None):
    """Largest |out - ref| a correct evaluation of R21-R23 may give, per output (binary64): the 16-bit
    sum's bound, one binary32 rounding of deq + acc16 (and one of the bias), then half an ulp of the
    output type at the result."""
    n_terms = len(d["O"]) if n_pad is None else n_pad
    e16 = gemm16_bound(n_terms, d["sum_abs16"])
    ref = np.abs(d["ref"])
    e32 = e16 + 2.0 ** -23 * (ref + e16)
    mag = ref + e32
    out = d["out_dtype"]
    if out == "f32":
        return e32
    # half an ulp of fp16 (11 significant bits, subnormal spacing 2^-24) or bf16 (8 significant bits)
    p, tiny = (11, 2.0 ** -24) if out == "f16" else (8, 2.0 ** -133)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.maximum(mag, tiny)))
    half_ulp = np.maximum(2.0 ** (e - p), tiny / 2)
    return e32 + half_ulp
