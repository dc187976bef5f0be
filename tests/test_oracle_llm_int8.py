"""Pins of the LLM.int8() decomposition oracle (CPU): the page's worked example, an exact-rational
brute force of the split, the threshold's edge, the two degenerate cases (no outlier: per-token
W8A8; every channel an outlier: the 16-bit product), the binary32 summation bound, and planted
mistakes that these pins catch."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import oracle.llm_int8 as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32
F64 = np.float64


def _fix1_row():
    with open(os.path.join(GOLDEN, "p3_fix1_outlier_row.json")) as f:
        g = json.load(f)
    k = g["row"]["k"]
    rng = np.random.default_rng(5)
    row = rng.uniform(g["row"]["ordinary_low"], g["row"]["ordinary_high"], k).astype(F32)
    row[0], row[1] = g["row"]["ordinary_high"], g["row"]["ordinary_low"]   # the stated range is reached
    for ch, v in g["row"]["outliers"].items():
        row[int(ch)] = v
    return g, row


def _fix1_checks(decompose):
    """The page's token: 4,096 values in [-2, 2] with channels 1512 = 45 and 2817 = -60. LLM.int8()
    sends those two channels (and the matching weights) through 16-bit; the other 4,094 get a step of
    2/127 ~ 0.016, 30 times finer than the 60/127 ~ 0.47 a single step for the row would take."""
    g, row = _fix1_row()
    pr = g["printed"]
    w = (np.random.default_rng(7).standard_normal((16, row.size)) * 0.02).astype(np.float16)
    d = decompose(row[None, :], "f32", O.NONE, w, w_dtype="f16")
    assert d["O"].tolist() == [1512, 2817]
    step = float(d["x_scale"][0])
    assert step == F32(2.0) / F32(127.0)
    assert abs(step - pr["step_without_outliers"]) < g["printed_precision"]["step_without_outliers"]
    assert float(F32(60.0) / F32(127.0)) / step == pytest.approx(pr["finer_factor"], rel=1e-6)
    assert d["xq"][0, 1512] == 0 and d["xq"][0, 2817] == 0
    assert np.abs(d["xq"][0].astype(int)).max() == 127               # the +-2 entries span the grid
    assert d["xo"][0].tolist() == [45.0, -60.0]                        # exact in fp16
    assert np.array_equal(d["wo"], w[:, [1512, 2817]].astype(F32))
    return d


def test_page3_example_one_token_through_a_layer():
    _fix1_checks(L.decompose)


# --------------------------------------------------------------------------- brute force of the split

def _exact_case(seed=0, m=3, k=8, n=5):
    """Inputs on which every rounding of the INT8 path is exact: each row's ordinary values are
    integer multiples of a power-of-two step with the largest magnitude 127 steps, each weight row
    likewise, and the outlier values and weights are fp16 numbers. Then deq + acc16 must equal the
    exact product X W^T."""
    rng = np.random.default_rng(seed)
    x = np.zeros((m, k), F32)
    for i in range(m):
        e = int(rng.integers(-8, -4))                                # 127 steps stay below 6
        codes = rng.integers(-127, 128, k).astype(F64)
        codes[0] = 127 * (1 if rng.random() < 0.5 else -1)           # channel 0 is never an outlier
        x[i] = (codes * 2.0 ** e).astype(F32)
    outl = [1, 5]
    x[:, outl] = rng.choice([-1, 1], (m, 2)) * rng.integers(800, 2000, (m, 2)) / 64.0   # |.| > 6, fp16-exact
    # keep every ordinary value below the threshold and the row maximum at 127 steps
    assert np.abs(np.delete(x, outl, axis=1)).max() < 6.0
    w = np.zeros((n, k), np.float16)
    for j in range(n):
        e = int(rng.integers(-9, -6))
        codes = rng.integers(-127, 128, k).astype(F64)
        codes[int(rng.integers(0, k))] = 127
        w[j] = (codes * 2.0 ** e).astype(np.float16)
    return x, w, outl


def _exact_product(x, w):
    xs = [[Fraction(float(v)) for v in r] for r in x]
    ws = [[Fraction(float(v)) for v in r] for r in np.asarray(w, F32)]
    return np.array([[float(sum(a * b for a, b in zip(xr, wr))) for wr in ws] for xr in xs])


@pytest.mark.parametrize("seed", range(4))
def test_split_sum_equals_the_exact_product(seed):
    x, w, outl = _exact_case(seed)
    d = L.decompose(x, "f32", O.NONE, w, w_dtype="f16")
    assert d["O"].tolist() == outl
    exact = _exact_product(x, w)
    assert np.array_equal(d["ref"], exact)                      # every rounding on this data is exact


def test_split_reproduces_xwt_in_binary64_on_random_data():
    # the split is a partition of the K sum: without quantisation both halves add up to X W^T
    rng = np.random.default_rng(3)
    y = rng.standard_normal((6, 64)).astype(F32)
    y[:, [7, 40]] *= 30
    w = rng.standard_normal((9, 64)).astype(F32)
    outl = L.outlier_channels(y)
    assert outl.tolist() == [7, 40]
    rest = np.setdiff1d(np.arange(64), outl)
    split = y[:, outl].astype(F64) @ w[:, outl].astype(F64).T + y[:, rest].astype(F64) @ w[:, rest].astype(F64).T
    assert np.allclose(split, y.astype(F64) @ w.astype(F64).T, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- threshold and degenerate cases

def test_threshold_is_inclusive():
    y = np.zeros((3, 64), F32)
    y[1, 10] = 6.0
    y[2, 11] = -6.0
    y[0, 12] = np.nextafter(F32(6.0), F32(0.0))
    y[2, 13] = -np.nextafter(F32(6.0), F32(0.0))
    assert L.outlier_channels(y).tolist() == [10, 11]
    assert L.outlier_channels(y, tau=0.0).tolist() == list(range(64))
    assert L.outlier_channels(y[:0]).tolist() == []


def test_no_outlier_reduces_to_per_token_w8a8():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((20, 256)) * 1.5).astype(np.float16)
    w = (rng.standard_normal((33, 256)) * 0.02).astype(np.float16)
    gamma = (1 + 0.1 * rng.standard_normal(256)).astype(F32)
    beta = (0.1 * rng.standard_normal(256)).astype(F32)
    d = L.decompose(x, "f16", O.LAYERNORM, w, gamma, beta, tau=np.inf)
    assert d["O"].size == 0
    q, s, _ = O.norm_quant(x, "f16", O.LAYERNORM, gamma, beta)      # no smoothing: the model's gamma, beta
    assert np.array_equal(d["xq"], q) and np.array_equal(d["x_scale"], s)
    wq, ws = O.quantize_rows(O.widen(w, "f16"))
    assert np.array_equal(d["wq"], wq) and np.array_equal(d["w_scale"], ws)
    _, deq = O.dequantize(O.int_gemm(q, wq), s, ws)
    assert not d["acc16"].any() and np.array_equal(d["ref"], deq.astype(F64))


def test_every_channel_an_outlier_gives_the_16bit_product():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 64)).astype(F32)                    # not fp16 numbers: the rounding shows
    w = rng.standard_normal((6, 64)).astype(F32)
    d = L.decompose(x, "f32", O.NONE, w, tau=0.0)
    assert d["O"].size == 64
    assert not d["xq"].any() and not d["x_scale"].any() and not d["deq"].any()
    x16 = x.astype(np.float16).astype(F32)
    w16 = w.astype(np.float16).astype(F32)
    assert np.allclose(d["ref"], _exact_product(x16, w16), rtol=2.0 ** -50, atol=0)
    assert not np.allclose(d["ref"], _exact_product(x, w), rtol=2.0 ** -30, atol=0)


def test_bf16_weights_take_the_bf16_format():
    rng = np.random.default_rng(13)
    x_bits = O.f32_to_bf16_bits(rng.standard_normal((3, 64)).astype(F32) * 10)
    w_bits = O.f32_to_bf16_bits(rng.standard_normal((5, 64)).astype(F32))
    d = L.decompose(x_bits, "bf16", O.RMSNORM, w_bits, tau=2.5)
    assert d["fmt"] == "bf16" and d["O"].size > 0
    xo_bits = O.f32_to_bf16_bits(d["y"][:, d["O"]])
    assert np.array_equal(d["xo"], O.widen(xo_bits, "bf16"))
    assert np.array_equal(d["wo"], O.widen(w_bits, "bf16")[:, d["O"]])


def test_accuracy_close_to_16bit_and_far_better_than_plain_int8():
    # the page: about 99.9% of the values go through INT8 and the accuracy matches 16-bit
    rng = np.random.default_rng(14)
    x = rng.standard_normal((64, 512)).astype(F32)
    x[:, [100, 300]] *= 50
    w = (rng.standard_normal((128, 512)) * 0.02).astype(F32)
    exact = x.astype(F64) @ w.astype(F64).T
    d = L.decompose(x, "f32", O.NONE, w)
    q, s = O.quantize_rows(x)
    wq, ws = O.quantize_rows(w)
    _, plain = O.dequantize(O.int_gemm(q, wq), s, ws)
    fp16 = x.astype(np.float16).astype(F64) @ w.astype(np.float16).astype(F64).T

    def rel(a):
        return np.linalg.norm(a - exact) / np.linalg.norm(exact)
    assert rel(d["ref"]) < 0.25 * rel(plain)
    assert rel(d["ref"]) < 20 * rel(fp16)


# --------------------------------------------------------------------------- binary32 summation bound

def test_gemm16_bound_covers_binary32_summations():
    rng = np.random.default_rng(15)
    for n_terms in (1, 7, 32, 41, 100, 300):
        a = rng.standard_normal((8, n_terms)).astype(np.float16).astype(F32) * 8
        b = rng.standard_normal((9, n_terms)).astype(np.float16).astype(F32)
        exact = L.gemm16(a, b)
        bound = L.gemm16_bound(n_terms, L.gemm16(np.abs(a), np.abs(b)))
        prods = a[:, None, :] * b[None, :, :]                         # exact in binary32
        seq = np.zeros((8, 9), F32)
        for i in range(n_terms):                                      # one order
            seq = seq + prods[:, :, i]
        rev = np.zeros((8, 9), F32)
        for i in reversed(range(n_terms)):                            # another
            rev = rev + prods[:, :, i]
        blk = np.zeros((8, 9), F32)
        for i0 in range(0, n_terms, 32):                              # 32-wide pairwise blocks
            p = prods[:, :, i0:i0 + 32]
            while p.shape[2] > 1:
                if p.shape[2] % 2:
                    p = np.concatenate([p, np.zeros_like(p[:, :, :1])], axis=2)
                p = p[:, :, 0::2] + p[:, :, 1::2]
            blk = blk + p[:, :, 0]
        for got in (seq, rev, blk):
            assert np.all(np.abs(got.astype(F64) - exact) <= bound)


def test_output_bound_covers_a_binary32_evaluation():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((16, 256)).astype(np.float16)
    x[:, [3, 77, 200]] = (x[:, [3, 77, 200]].astype(F32) * 40).astype(np.float16)
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float16)
    for out in ("f32", "f16", "bf16"):
        d = L.decompose(x, "f16", O.NONE, w, out_dtype=out)
        acc16_32 = (d["xo"][:, None, :] * d["wo"][None, :, :]).sum(axis=2, dtype=F32)
        out32 = (d["deq"] + acc16_32).astype(F32)
        got = O.round_output(out32, out)
        got64 = (got.astype(np.uint32) << 16).view(F32).astype(F64) if out == "bf16" else got.astype(F64)
        assert np.all(np.abs(got64 - d["ref"]) <= L.output_bound(d))


# --------------------------------------------------------------------------- planted mistakes

def _mutant(**changes):
    """decompose with one step changed."""
    def run(x, dtype, norm, w, gamma=None, beta=None, eps=1e-5, tau=L.TAU, w_dtype=None, wq=None, w_scale=None,
            bias=None, out_dtype="f32"):
        w_dtype = w_dtype or dtype
        y, _ = L.activations(x, dtype, norm, gamma, beta, eps)
        outl = changes.get("outliers", L.outlier_channels)(y, tau)
        y_int = y.copy()
        if not changes.get("keep_outlier_codes"):
            y_int[:, outl] = 0
        xq, xs = O.quantize_rows(y if changes.get("step_over_all") else y_int)
        if changes.get("step_over_all"):
            xq[:, outl] = 0
        wq, w_scale = L.weights(w, w_dtype)
        _, deq = O.dequantize(O.int_gemm(xq, wq), xs, w_scale)
        fmt = L.half_format(w_dtype)
        xo = y[:, outl] if changes.get("no_16bit_rounding") else L.round16(y[:, outl], fmt)
        w32 = O.widen(w, w_dtype)
        wo = L.round16(w32[outl, :].T if changes.get("weight_rows") else w32[:, outl], fmt)
        acc16 = L.gemm16(xo, wo)
        return {"y": y, "O": outl, "xq": xq, "x_scale": xs, "deq": deq, "xo": xo, "wo": wo, "acc16": acc16,
                "ref": deq.astype(F64) + acc16}
    return run


def test_planted_mistakes_are_caught():
    strict = _mutant(outliers=lambda y, tau: np.where(np.max(np.abs(y), axis=0) > F32(tau))[0])
    with pytest.raises(AssertionError):
        y = np.zeros((2, 64), F32)
        y[0, 10] = 6.0
        assert strict(y, "f32", O.NONE, np.ones((3, 64), F32))["O"].tolist() == [10]
    with pytest.raises(AssertionError):                                      # step over the outliers too
        _fix1_checks(_mutant(step_over_all=True))
    x, w, outl = _exact_case(0, k=8, n=8)                                    # square, so a row gather runs
    exact = _exact_product(x, w)
    for bad in (_mutant(keep_outlier_codes=True), _mutant(weight_rows=True)):
        assert not np.array_equal(bad(x, "f32", O.NONE, w, w_dtype="f16")["ref"], exact)
    rng = np.random.default_rng(12)
    xr = rng.standard_normal((4, 64)).astype(F32)
    wr = rng.standard_normal((6, 64)).astype(F32)
    d = _mutant(no_16bit_rounding=True)(xr, "f32", O.NONE, wr, tau=0.0)
    x16, w16 = xr.astype(np.float16).astype(F32), wr.astype(np.float16).astype(F32)
    assert not np.allclose(d["ref"], _exact_product(x16, w16), rtol=2.0 ** -50, atol=0)
