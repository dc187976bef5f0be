"""Plain, slow CPU oracle of the SmoothQuant W8A8 linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. Written from the pages,
with numpy and the Python standard library; it shares no code with the HIP path.

What it follows (page title, then section):

* "LLM.int8() and SmoothQuant" -- "Fix 2: move the difficulty into the weights"
  and "going deeper / SmoothQuant": for positive per-input-channel factors s,
  Y = X W = (X diag(s)^-1)(diag(s) W) with X tokens x channels and W channels x
  outputs, s_j = max_t|X_tj|^alpha / max_k|W_jk|^(1-alpha), max_t|X_tj| taken on
  calibration data; X-hat is then quantised per token, W-hat per channel.
  "Fix 1" / "example: one token through a layer": a per-row INT8 step is the
  row's largest magnitude divided by 127.
* "SmoothQuant, in depth" -- "The calibration data flow" and its code: a running
  per-input-channel max of |input| over every calibration token; eps = 1e-5
  clamps on act_max, on w_max and on s; the norm weight (and bias) divided by s,
  each weight column multiplied by s. "Where the scales go in a decoder block":
  projections fed by one norm share one s built from the elementwise max of
  their weight maxima. "Granularity: O1, O2, O3 and what kernels run today":
  per-output-channel weight scales, per-token dynamic activation scales, an INT32
  accumulator, epilogue out = acc * scale_token[i] * scale_channel[j], then
  conversion to FP16/BF16.

Readings where the pages leave a step open:

R1  step = fl32(absmax / 127); code = clip(round_half_even(fl32(v / step)),
    -127, 127); a zero step gives all-zero codes.
R2  norm statistics (LayerNorm mean and variance, RMSNorm mean square) are
    exact rationals rounded once to binary32; rstd = fl32(1 / fl32(sqrt(fl32(var + eps)))).
R3  every later elementwise step is a single binary32 operation rounded on its
    own, in the order written (no fused multiply-add).
R4  s_j is the real value a'^alpha / w'^(1 - alpha) rounded once to binary32,
    a' = max(a_j, eps), w' = max(w_j, eps), then s_j = max(s_j, eps); the
    exponent 1 - alpha is the binary64 difference. gamma' = fl32(gamma / s),
    beta' = fl32(beta / s); with no norm in front, the fold target is a
    per-channel multiplier gamma' = fl32(1 / s).
R5  calibration records |y| of the fp32 activations the quantiser would see
    (the norm applied with the unfolded gamma, beta).
R6  the GEMM epilogue is fl32(fl32(fl32(acc) * x_scale[m]) * w_scale[n]),
    plus an optional bias fl32(. + b[n]), then round-half-even to the output type.
R14 per-tensor granularity ("SmoothQuant, in depth", "Granularity: O1, O2, O3":
    per-tensor weights at every level, a static activation scale at O3; the
    level table itself is lost): O2 takes one dynamic step for the whole
    activation tensor, fl32(max |y| / 127) over every element; O3 a static step
    fixed at calibration; per-tensor weights one step for the whole W-hat.
    Codes follow R1, clipping included (values beyond a static step's range
    clip, as the page's failure-mode note on static scales says). The per-row
    and per-channel scale vectors the GEMM reads hold the step repeated, so
    R6 is unchanged.
R16 the FP8 variant ("SmoothQuant -- interactive paper explainer", timeline
    "2023+ The efficiency stack" and "What it did NOT solve"; "LLM.int8() and
    SmoothQuant", "example: what you get": FP8 W8A8 took over the INT8 role and
    kept the smoothing): codes are OCP E4M3 (bias 7, 3 mantissa
    bits, largest finite 448, no infinities, S.1111.111 is NaN); a per-row step
    is fl32(absmax / 448) and a code is the round-half-even E4M3 value of
    fl32(v / step). Magnitudes above 448 round to NaN past the 464 midpoint
    (448 at the midpoint, ties to even); quotients here never exceed
    448 * (1 + 2^-23). The GEMM multiplies decoded codes: every product is
    exact, and the oracle's binary64 sum is exact for K <= 2^17; a binary32
    accumulator in another order differs by a bounded amount (gemm_fp8_bound).
R15 the static activation step is fl32(max_j fl32(a_j / s_j) / 127): the
    smoothed input of channel j is y_j / s_j, so its calibration maximum is
    a_j / s_j (a_j from R5, s_j from R4).
R18 FP8 with one step for the whole tensor (R14's granularities with R16's
    codes): the dynamic step is fl32(max |y| / 448), the static one
    fl32(max_j fl32(a_j / s_j) / 448) (R15), and the quotient fl32(v / step) is
    saturated to [-448, 448] before encoding, as INT8 codes clip to +-127: a
    value beyond the step's range takes the largest code, never NaN.

Where a step rounds a real number that the oracle computes exactly (R2, R4),
it also reports how far that number lies from the binary32 rounding boundary,
in units of the binary32 spacing. A different correct evaluation (a GPU's fp64
sum or pow) can land on the other side only when that distance is tiny; the
tests accept either neighbour for such near-ties and check the rest against it.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

__all__ = [
    "NONE", "LAYERNORM", "RMSNORM", "QMAX", "EPS_FOLD",
    "widen", "f32_to_bf16_bits", "round_output", "rn32_rational",
    "row_stats", "normalize", "quantize_rows", "norm_quant", "norm_quant_row_variants", "row_y_variants",
    "calibrate", "weight_colmax", "smoothing_factors", "fold",
    "int_gemm", "int_gemm_loops", "dequantize", "w8a8_linear",
    "quantize_tensor", "norm_quant_per_tensor", "static_step", "fold_per_tensor",
    "E4M3_MAX", "e4m3_encode", "e4m3_decode", "quantize_rows_fp8", "norm_quant_fp8", "fold_fp8", "gemm_fp8",
    "gemm_fp8_bound", "quantize_tensor_fp8", "norm_quant_fp8_per_tensor", "static_step_fp8",
    "fold_fp8_per_tensor",
]

F32 = np.float32
NONE, LAYERNORM, RMSNORM = "none", "layernorm", "rmsnorm"
QMAX = 127
EPS_FOLD = 1e-5
NEAR_TIE = 2.0 ** -12       # distance (binary32 spacings) below which a rounding is a near-tie


# --------------------------------------------------------------------------- O0 number formats

def widen(x, dtype: str) -> np.ndarray:
    """Stored values as binary32: fp16 widens exactly; bf16 (uint16 bits) is bits << 16."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def f32_to_bf16_bits(v) -> np.ndarray:
    """binary32 -> bfloat16 bit pattern, round half to even (finite inputs)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def round_output(v32: np.ndarray, out_dtype: str) -> np.ndarray:
    """Final conversion of binary32 results: identity, fp16 (numpy casts half-to-even) or bf16 bits."""
    if out_dtype == "f32":
        return v32.astype(np.float32)
    if out_dtype == "f16":
        return v32.astype(np.float16)
    if out_dtype == "bf16":
        return f32_to_bf16_bits(v32)
    raise ValueError(f"unknown output dtype {out_dtype}")


def rn32_rational(num: int, den: int):
    """Nearest binary32 to the rational num/den (den > 0), ties to even.

    Returns (value, dist, other): `other` is the neighbour on the far side of
    the rounding boundary and `dist` the distance from num/den to that boundary
    in binary32 spacings (0 on a midpoint, 0.5 when num/den is representable).
    """
    if num == 0:
        return F32(0.0), 0.5, F32(0.0)
    sign = -1 if num < 0 else 1
    a = abs(num)
    t = a.bit_length() - den.bit_length()          # floor(log2(a/den)) is t or t - 1
    if (a << max(0, -t)) < (den << max(0, t)):
        t -= 1
    e = max(t - 23, -149)                          # spacing 2^e: 24 significant bits, or subnormal
    n_, d_ = (a << -e, den) if e < 0 else (a, den << e)
    q, r = divmod(n_, d_)
    up = 2 * r > d_ or (2 * r == d_ and (q & 1))
    near, far = (q + 1, q) if up else (q, q + 1)
    dist = float(abs(Fraction(2 * r - d_, 2 * d_)))
    return F32(sign * math.ldexp(near, e)), dist, F32(sign * math.ldexp(far, e))


def _scaled_ints(v32: np.ndarray):
    """Exact integers n with v32 == n * 2**e0 (Python ints, so sums and squares stay exact)."""
    mant, ex = np.frexp(v32.astype(np.float64))
    m = (mant * float(1 << 24)).astype(np.int64)   # every binary32 significand fits 24 bits
    e = ex.astype(np.int64) - 24
    nz = m != 0
    if not nz.any():
        return [0] * v32.size, 0
    e0 = int(e[nz].min())
    sh = (e - e0).tolist()
    return [int(mi) << si if mi else 0 for mi, si in zip(m.tolist(), sh)], e0


def _ratio(num: int, exp2: int, den: int):
    return (num << exp2, den) if exp2 >= 0 else (num, den << -exp2)


# --------------------------------------------------------------------------- O3 norm + quantise

def row_stats(x32_row: np.ndarray, norm: str) -> dict:
    """Exact statistics of one fp32 row, each rounded once to binary32 (reading R2).

    LayerNorm: mean = sum(x)/K, var = sum((x - mean)^2)/K = (K*sum(x^2) - sum(x)^2)/K^2.
    RMSNorm:   var = sum(x^2)/K (no centring).
    """
    k = x32_row.size
    n, e0 = _scaled_ints(x32_row)
    s2 = sum(v * v for v in n)
    if norm == LAYERNORM:
        s1 = sum(n)
        mu, mu_d, mu_o = rn32_rational(*_ratio(s1, e0, k))
        var, var_d, var_o = rn32_rational(*_ratio(k * s2 - s1 * s1, 2 * e0, k * k))
    elif norm == RMSNORM:
        mu, mu_d, mu_o = F32(0.0), 0.5, F32(0.0)
        var, var_d, var_o = rn32_rational(*_ratio(s2, 2 * e0, k))
    else:
        raise ValueError(norm)
    return {"mu": mu, "mu_dist": mu_d, "mu_other": mu_o,
            "var": var, "var_dist": var_d, "var_other": var_o}


def normalize(x32, norm, mu=None, var=None, gamma=None, beta=None, eps=1e-5) -> np.ndarray:
    """y of the fused kernel, one binary32 rounding per operation (reading R3).

    LayerNorm: y = ((x - mu) * rstd) * gamma + beta;  RMSNorm: y = (x * rstd) * gamma;
    none: y = x * gamma (gamma absent -> y = x). A missing gamma/beta means 1/0.
    """
    x32 = np.atleast_2d(np.asarray(x32, dtype=F32))
    if norm == NONE:
        return x32 * np.asarray(gamma, F32)[None, :] if gamma is not None else x32.copy()
    var = np.asarray(var, F32).reshape(-1, 1)
    r = F32(1.0) / np.sqrt(var + F32(eps))
    if norm == LAYERNORM:
        y = (x32 - np.asarray(mu, F32).reshape(-1, 1)) * r
    elif norm == RMSNORM:
        y = x32 * r
    else:
        raise ValueError(norm)
    if gamma is not None:
        y = y * np.asarray(gamma, F32)[None, :]
    if norm == LAYERNORM and beta is not None:
        y = y + np.asarray(beta, F32)[None, :]
    return y


def quantize_rows(y: np.ndarray):
    """Symmetric INT8 with one step per row: step = absmax/127, codes half-to-even (reading R1)."""
    y = np.atleast_2d(np.asarray(y, dtype=F32))
    amax = np.max(np.abs(y), axis=1) if y.shape[1] else np.zeros(y.shape[0], F32)
    step = amax / F32(QMAX)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = y / step[:, None]
    q = np.clip(np.rint(t), -QMAX, QMAX)
    q[step == 0] = 0
    return q.astype(np.int8), step.astype(F32)


def _stats_block(x32, norm):
    m = x32.shape[0]
    mu = np.zeros(m, F32)
    var = np.zeros(m, F32)
    tie = np.zeros(m, bool)
    alt = {}
    for i in range(m):
        st = row_stats(x32[i], norm)
        mu[i], var[i] = st["mu"], st["var"]
        if min(st["mu_dist"], st["var_dist"]) < NEAR_TIE:
            tie[i] = True
            alt[i] = st
    return mu, var, tie, alt


def norm_quant(x, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5):
    """Runtime activation path: norm with folded gamma', beta', then per-token INT8.

    Returns (codes int8 [M,K], x_scale fp32 [M], info); info["near_tie"] marks
    rows whose statistics sit within NEAR_TIE of a binary32 boundary.
    """
    x32 = widen(x, dtype)
    if norm == NONE:
        y = normalize(x32, NONE, gamma=gamma_f)
        info = {"near_tie": np.zeros(x32.shape[0], bool), "alt": {}}
    else:
        mu, var, tie, alt = _stats_block(x32, norm)
        y = normalize(x32, norm, mu, var, gamma_f, beta_f, eps)
        info = {"mu": mu, "var": var, "near_tie": tie, "alt": alt}
    q, step = quantize_rows(y)
    info["y"] = y
    return q, step, info


def row_y_variants(x_row, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5):
    """y of one row [1, K] for every correct rounding of its statistics (reading R2).

    A statistic within NEAR_TIE of a binary32 rounding boundary may round to
    either neighbour; every combination of the mean's and the variance's
    admissible roundings gives one y. A row without a near-tie gives one y.
    """
    x32 = widen(np.asarray(x_row)[None, :], dtype)
    if norm == NONE:
        return [normalize(x32, NONE, gamma=gamma_f)]
    st = row_stats(x32[0], norm)
    mus = {float(st["mu"])} | ({float(st["mu_other"])} if st["mu_dist"] < NEAR_TIE else set())
    vrs = {float(st["var"])} | ({float(st["var_other"])} if st["var_dist"] < NEAR_TIE else set())
    return [normalize(x32, norm, [mu], [var], gamma_f, beta_f, eps) for mu in sorted(mus) for var in sorted(vrs)]


def norm_quant_row_variants(x_row, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5):
    """Every (codes, step) a correct evaluation may give for one row whose statistics are near-ties."""
    return [quantize_rows(y) for y in row_y_variants(x_row, dtype, norm, gamma_f, beta_f, eps)]


# --------------------------------------------------------------------------- O1 calibration

def calibrate(x, dtype, norm, gamma=None, beta=None, eps=1e-5, absmax=None):
    """Running per-input-channel max of |y| over calibration tokens (reading R5).

    ("SmoothQuant, in depth", "The calibration data flow": every token of every
    calibration sequence, a running elementwise max across batches.)
    Returns (absmax fp32 [K], info) with per-row near-tie flags as in norm_quant.
    """
    x32 = widen(x, dtype)
    if norm == NONE:
        y = x32
        info = {"near_tie": np.zeros(x32.shape[0], bool), "alt": {}}
    else:
        mu, var, tie, alt = _stats_block(x32, norm)
        y = normalize(x32, norm, mu, var, gamma, beta, eps)
        info = {"mu": mu, "var": var, "near_tie": tie, "alt": alt}
    a = np.max(np.abs(y), axis=0).astype(F32)
    if absmax is not None:
        a = np.maximum(np.asarray(absmax, F32), a)
    info["y"] = y
    return a, info


# --------------------------------------------------------------------------- O2 smoothing factors and fold

def weight_colmax(w, dtype, block: int = 4096) -> np.ndarray:
    """w_j = max over output rows n of |W[n, j]| for a torch-layout [N, K] weight (in row blocks)."""
    w = np.asarray(w)
    out = np.zeros(w.shape[1], F32)
    for n0 in range(0, w.shape[0], block):
        out = np.maximum(out, np.max(np.abs(widen(w[n0:n0 + block], dtype)), axis=0))
    return out.astype(F32)


def _s_exact(a: float, w: float, alpha: float):
    """a^alpha / w^(1-alpha) to 60 significant digits, rounded once to binary32."""
    with localcontext() as ctx:
        ctx.prec = 60
        v = (Decimal(a) ** Decimal(alpha)) / (Decimal(w) ** Decimal(1.0 - alpha))
    f = Fraction(v)
    return rn32_rational(f.numerator, f.denominator)


def smoothing_factors(act_absmax, w_colmax, alpha: float, eps: float = EPS_FOLD):
    """s_j = max(a_j, eps)^alpha / max(w_j, eps)^(1-alpha), clamped below at eps (reading R4).

    A binary64 evaluation errs by a few binary64 ulps, which decides the binary32
    rounding unless the value sits near a binary32 midpoint; such channels are
    re-evaluated in 60-digit decimal arithmetic.
    Returns (s fp32 [K], dist [K], other fp32 [K]).
    """
    a1 = np.maximum(np.asarray(act_absmax, F32), F32(eps))
    w1 = np.maximum(np.asarray(w_colmax, F32), F32(eps))
    k = a1.size
    s = np.empty(k, F32)
    dist = np.empty(k)
    other = np.empty(k, F32)
    for j, (aj, wj) in enumerate(zip(a1.tolist(), w1.tolist())):
        v64 = math.pow(aj, alpha) / math.pow(wj, 1.0 - alpha)
        f = Fraction(v64)
        val, d, o = rn32_rational(f.numerator, f.denominator)
        if d < 2.0 ** -16:
            val, d, o = _s_exact(aj, wj, alpha)
        s[j], dist[j], other[j] = val, d, o
    clamped = s < F32(eps)
    s = np.maximum(s, F32(eps))
    dist[clamped] = 0.5
    return s, dist, other


def fold(act_absmax, w, dtype, alpha, eps=EPS_FOLD, norm=NONE, gamma=None, beta=None, s=None):
    """Offline smoothing: s, folded norm params and per-output-channel INT8 weights.

    W-hat[n, j] = fl32(W[n, j] * s_j) (each input column scaled by s_j), then one
    INT8 step per output row (quantize_rows). gamma' = gamma / s, beta' = beta / s;
    with no norm, gamma' = 1 / s is the multiplier the activation quantiser applies.
    Passing `s` skips the factor computation (to continue from another correct s).
    """
    w32 = widen(w, dtype)
    wmax = np.max(np.abs(w32), axis=0).astype(F32)
    dist = other = None
    if s is None:
        s, dist, other = smoothing_factors(act_absmax, wmax, alpha, eps)
    s = np.asarray(s, F32)
    w_hat = w32 * s[None, :]
    wq, w_scale = quantize_rows(w_hat)
    if norm == NONE or gamma is None:
        gamma_f = F32(1.0) / s
    else:
        gamma_f = np.asarray(gamma, F32) / s
    beta_f = np.asarray(beta, F32) / s if (norm == LAYERNORM and beta is not None) else None
    return {"s": s, "s_dist": dist, "s_other": other, "w_colmax": wmax,
            "gamma_f": gamma_f.astype(F32), "beta_f": None if beta_f is None else beta_f.astype(F32),
            "wq": wq, "w_scale": w_scale, "w_hat": w_hat}


# --------------------------------------------------------------------------- per-tensor granularities (R14, R15)

def quantize_tensor(y, step=None):
    """One INT8 step for a whole tensor (reading R14).

    step None: the dynamic step fl32(max |y| / 127) over every element (O2, and
    per-tensor weights); otherwise the given static step (O3). Codes are
    clip(round_half_even(fl32(y / step)), -127, 127); a step that is not
    positive gives all-zero codes. Returns (codes int8, step fp32 scalar).
    """
    y = np.atleast_2d(np.asarray(y, dtype=F32))
    if step is None:
        amax = np.max(np.abs(y)) if y.size else F32(0)
        step = F32(amax) / F32(QMAX)
    step = F32(step)
    if not step > 0:
        return np.zeros(y.shape, np.int8), step
    q = np.clip(np.rint(y / step), -QMAX, QMAX)
    return q.astype(np.int8), step


def norm_quant_per_tensor(x, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5, step=None):
    """Norm with the folded gamma', beta' (exactly as norm_quant), then one step for the tensor.

    step None: per-tensor dynamic (O2); a number: the static calibrated step (O3).
    Returns (codes int8 [M,K], x_scale fp32 [M] = the step repeated, info) with
    info["near_tie"] as in norm_quant.
    """
    x32 = widen(x, dtype)
    if norm == NONE:
        y = normalize(x32, NONE, gamma=gamma_f)
        info = {"near_tie": np.zeros(x32.shape[0], bool), "alt": {}}
    else:
        mu, var, tie, alt = _stats_block(x32, norm)
        y = normalize(x32, norm, mu, var, gamma_f, beta_f, eps)
        info = {"mu": mu, "var": var, "near_tie": tie, "alt": alt}
    q, st = quantize_tensor(y, step)
    info["y"] = y
    return q, np.full(x32.shape[0], st, F32), info


def static_step(act_absmax, s):
    """Static per-tensor activation step from calibration (reading R15): fl32(max_j fl32(a_j / s_j) / 127)."""
    r = np.asarray(act_absmax, F32) / np.asarray(s, F32)
    return F32(np.max(r) if r.size else F32(0)) / F32(QMAX)


def fold_per_tensor(act_absmax, w, dtype, alpha, eps=EPS_FOLD, norm=NONE, gamma=None, beta=None, s=None):
    """fold() with one weight step for the whole W-hat (reading R14): w_scale holds it repeated."""
    f = fold(act_absmax, w, dtype, alpha, eps, norm, gamma, beta, s)
    wq, st = quantize_tensor(f["w_hat"])
    f["wq"] = wq
    f["w_scale"] = np.full(f["w_hat"].shape[0], st, F32)
    return f


# --------------------------------------------------------------------------- FP8 (OCP E4M3) variant (R16)

E4M3_MAX = 448.0


def e4m3_encode(v) -> np.ndarray:
    """binary32 values -> OCP E4M3 codes (uint8), round half to even (reading R16).

    Normal range |v| >= 2^-6: v = m * 2^e with m in [1, 2); the code keeps
    round_half_even((m - 1) * 8) as its 3-bit mantissa (a carry to 8 moves to
    the next exponent) under the biased exponent e + 7. Below 2^-6 the spacing
    is the subnormal 2^-9. Every step is exact in binary64, and numpy's rint
    rounds half to even. Codes past 0x7E (448) are NaN (0x7F, with the sign).
    """
    v = np.asarray(v, dtype=F32)
    a = np.abs(v).astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    sub = a < 2.0 ** -6
    q_sub = np.rint(a * 2.0 ** 9).astype(np.int64)                  # 0 .. 8 (8 is the smallest normal, 0x08)
    frac, exp = np.frexp(np.where(sub, 1.0, a))                      # a = frac * 2^exp, frac in [0.5, 1)
    e = exp.astype(np.int64) - 1
    mant = np.rint((frac * 2.0 - 1.0) * 8.0).astype(np.int64)
    e = np.where(mant == 8, e + 1, e)
    mant = np.where(mant == 8, 0, mant)
    q_norm = (e + 7) * 8 + mant
    q = np.where(sub, q_sub, q_norm)
    q = np.where((q > 0x7E) | np.isnan(a), 0x7F, q)
    return (q | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 codes -> binary32 values (exact); 0x7F / 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    ex, mant = mag >> 3, mag & 7
    val = np.where(ex == 0, mant * 2.0 ** -9, (1.0 + mant / 8.0) * np.exp2(ex - 7.0))
    val = np.where(mag == 0x7F, np.nan, val)
    return np.where(c & 0x80, -val, val).astype(F32)


def quantize_rows_fp8(y: np.ndarray):
    """One FP8 step per row: step = fl32(absmax / 448), codes E4M3(fl32(y / step)); a zero step gives 0."""
    y = np.atleast_2d(np.asarray(y, dtype=F32))
    amax = np.max(np.abs(y), axis=1) if y.shape[1] else np.zeros(y.shape[0], F32)
    step = (amax / F32(E4M3_MAX)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (y / step[:, None]).astype(F32)
    t[step == 0] = 0
    return e4m3_encode(t), step


def norm_quant_fp8(x, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5):
    """norm_quant with FP8 (E4M3) codes and steps fl32(absmax / 448)."""
    x32 = widen(x, dtype)
    if norm == NONE:
        y = normalize(x32, NONE, gamma=gamma_f)
        info = {"near_tie": np.zeros(x32.shape[0], bool), "alt": {}}
    else:
        mu, var, tie, alt = _stats_block(x32, norm)
        y = normalize(x32, norm, mu, var, gamma_f, beta_f, eps)
        info = {"mu": mu, "var": var, "near_tie": tie, "alt": alt}
    q, step = quantize_rows_fp8(y)
    info["y"] = y
    return q, step, info


def fold_fp8(act_absmax, w, dtype, alpha, eps=EPS_FOLD, norm=NONE, gamma=None, beta=None, s=None):
    """fold() with FP8 (E4M3) weight codes, one step fl32(max|W-hat row| / 448) per output row."""
    f = fold(act_absmax, w, dtype, alpha, eps, norm, gamma, beta, s)
    f["wq"], f["w_scale"] = quantize_rows_fp8(f["w_hat"])
    return f


def gemm_fp8(xq, wq, block: int = 512) -> np.ndarray:
    """acc[m, n] = sum_k dec(xq[m, k]) * dec(wq[n, k]) exactly (binary64: products of two E4M3
    values are exact, and their sums are multiples of 2^-18 below 2^35 for K <= 2^17)."""
    a = e4m3_decode(xq).astype(np.float64)
    b = e4m3_decode(wq).astype(np.float64)
    out = np.empty((a.shape[0], b.shape[0]), np.float64)
    for i in range(0, a.shape[0], block):
        out[i:i + block] = a[i:i + block] @ b.T
    return out


def gemm_fp8_bound(xq, wq, k_step: int = 128) -> np.ndarray:
    """Bound on |acc_gpu - acc| for a binary32 accumulation in any order: each of the K/k_step
    accumulation steps plus a log2(k_step)-deep tree inside one step rounds once, so the error is
    at most n * 2^-24 * sum_k |x_k w_k| (first order, n = K/k_step + log2(k_step) + 2)."""
    a = np.abs(e4m3_decode(xq).astype(np.float64))
    b = np.abs(e4m3_decode(wq).astype(np.float64))
    k = a.shape[1]
    n = -(-k // k_step) + int(math.log2(k_step)) + 2
    return n * 2.0 ** -24 * (a @ b.T)


def quantize_tensor_fp8(y, step=None):
    """One FP8 step for a whole tensor (reading R18).

    step None: the dynamic step fl32(max |y| / 448) over every element; otherwise
    the given static step. Codes are E4M3(clip(fl32(y / step), -448, 448)), the
    clip saturating values beyond the step's range; a step that is not positive
    gives all-zero codes. Returns (codes uint8, step fp32 scalar).
    """
    y = np.atleast_2d(np.asarray(y, dtype=F32))
    if step is None:
        amax = np.max(np.abs(y)) if y.size else F32(0)
        step = F32(amax) / F32(E4M3_MAX)
    step = F32(step)
    if not step > 0:
        return np.zeros(y.shape, np.uint8), step
    with np.errstate(over="ignore"):
        t = (y / step).astype(F32)
    t = np.clip(t, F32(-E4M3_MAX), F32(E4M3_MAX))
    return e4m3_encode(t), step


def norm_quant_fp8_per_tensor(x, dtype, norm, gamma_f=None, beta_f=None, eps=1e-5, step=None):
    """norm_quant_per_tensor with FP8 codes: one dynamic (step None) or static step for the tensor."""
    x32 = widen(x, dtype)
    if norm == NONE:
        y = normalize(x32, NONE, gamma=gamma_f)
        info = {"near_tie": np.zeros(x32.shape[0], bool), "alt": {}}
    else:
        mu, var, tie, alt = _stats_block(x32, norm)
        y = normalize(x32, norm, mu, var, gamma_f, beta_f, eps)
        info = {"mu": mu, "var": var, "near_tie": tie, "alt": alt}
    q, st = quantize_tensor_fp8(y, step)
    info["y"] = y
    return q, np.full(x32.shape[0], st, F32), info


def static_step_fp8(act_absmax, s):
    """Static per-tensor FP8 activation step (reading R18): fl32(max_j fl32(a_j / s_j) / 448)."""
    r = np.asarray(act_absmax, F32) / np.asarray(s, F32)
    return F32(np.max(r) if r.size else F32(0)) / F32(E4M3_MAX)


def fold_fp8_per_tensor(act_absmax, w, dtype, alpha, eps=EPS_FOLD, norm=NONE, gamma=None, beta=None, s=None):
    """fold() with FP8 weight codes and one step fl32(max |W-hat| / 448) for the whole W-hat (R18)."""
    f = fold(act_absmax, w, dtype, alpha, eps, norm, gamma, beta, s)
    wq, st = quantize_tensor_fp8(f["w_hat"])
    f["wq"] = wq
    f["w_scale"] = np.full(f["w_hat"].shape[0], st, F32)
    return f


# --------------------------------------------------------------------------- O4 GEMM and epilogue

def int_gemm(xq, wq, block: int = 512) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * wq[n, k], exactly.

    Every product is at most 127^2 and every partial sum an integer of
    magnitude below 2^53, so a binary64 matrix product of the int8 values is
    exact whatever order the library sums in.
    """
    xq = np.asarray(xq)
    wq64 = np.asarray(wq).astype(np.float64)
    m = xq.shape[0]
    acc = np.empty((m, wq64.shape[0]), np.int64)
    for m0 in range(0, m, block):
        acc[m0:m0 + block] = (xq[m0:m0 + block].astype(np.float64) @ wq64.T).astype(np.int64)
    return acc


def int_gemm_loops(xq, wq) -> np.ndarray:
    """Brute-force integer triple loop (tiny shapes only)."""
    xs, ws = np.asarray(xq).tolist(), np.asarray(wq).tolist()
    return np.array([[sum(a * b for a, b in zip(xr, wr)) for wr in ws] for xr in xs], dtype=np.int64)


def dequantize(acc, x_scale, w_scale, bias=None, out_dtype="f32"):
    """out = cvt(fl32(fl32(fl32(acc) * x_scale[m]) * w_scale[n]) (+ bias[n])) (reading R6).

    Returns (out in out_dtype storage, binary32 value before the final conversion).
    """
    v = np.asarray(acc).astype(F32)
    v = v * np.asarray(x_scale, F32)[:, None]
    v = v * np.asarray(w_scale, F32)[None, :]
    if bias is not None:
        v = v + np.asarray(bias, F32)[None, :]
    return round_output(v, out_dtype), v


def w8a8_linear(x, x_cal, w, dtype, norm, alpha, gamma=None, beta=None, eps=1e-5,
                out_dtype="f32", bias=None):
    """The whole layer: calibrate -> fold -> norm+quantise -> INT8 GEMM -> epilogue."""
    a, _ = calibrate(x_cal, dtype, norm, gamma, beta, eps)
    f = fold(a, w, dtype, alpha, EPS_FOLD, norm, gamma, beta)
    xq, xs, _ = norm_quant(x, dtype, norm, f["gamma_f"], f["beta_f"], eps)
    acc = int_gemm(xq, f["wq"])
    out, v32 = dequantize(acc, xs, f["w_scale"], bias, out_dtype)
    return {"absmax": a, **f, "xq": xq, "x_scale": xs, "acc": acc, "out": out, "out32": v32}
