"""Pins of the oracle's FP8 (OCP E4M3) variant to facts fixed outside it: the format's own
definition (hand-encoded values, every code's round trip, midpoints to even), torch's
independent float8_e4m3fn cast, quantiser invariants, and exact-rational brute force of the
FP8 GEMM with its accumulation bound. CPU only."""
from fractions import Fraction

import numpy as np
import torch

import oracle as O

F32 = np.float32


def test_e4m3_hand_encoded_values():
    # sign | 4-bit exponent (bias 7) | 3-bit mantissa; subnormals at 2^-9 spacing
    cases = {1.0: 0x38, 2.0: 0x40, 0.5: 0x30, -1.0: 0xB8, 448.0: 0x7E, 416.0: 0x7D, 2.0 ** -9: 0x01,
             2.0 ** -6: 0x08, 7 * 2.0 ** -9: 0x07, 0.0: 0x00, 1.125: 0x39, 240.0: 0x77, 3.0: 0x44,
             1.0625: 0x38, 1.1875: 0x3A, 17.0: 0x58, 19.0: 0x5A, 464.0: 0x7E, 2.0 ** -10: 0x00}
    v = np.array(list(cases), F32)
    assert [int(c) for c in O.e4m3_encode(v)] == list(cases.values())
    assert int(O.e4m3_encode(np.array([-0.0], F32))[0]) == 0x80
    assert int(O.e4m3_encode(np.array([465.0], F32))[0]) == 0x7F                    # past the 464 midpoint: NaN
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_every_code_round_trips_and_midpoints_go_to_even():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = O.e4m3_decode(codes)
    assert np.array_equal(O.e4m3_encode(vals), codes)
    pos = np.sort(O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64))
    assert np.all(np.diff(pos) > 0)                                                  # monotone
    mids = ((pos[:-1] + pos[1:]) / 2).astype(F32)                                    # exact in binary32
    got = O.e4m3_encode(mids)
    want = np.where(np.arange(len(mids)) % 2 == 0, np.arange(len(mids)), np.arange(1, len(mids) + 1))
    assert np.array_equal(got.astype(np.int64), want)                               # the even code of the pair


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-4, 3, 50000),
                        rng.uniform(-460, 460, 20000)]).astype(F32)
    v = v[np.abs(v) <= 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), ref)


def test_quantize_rows_fp8_invariants():
    rng = np.random.default_rng(4)
    y = (rng.standard_normal((20, 300)) * np.exp(rng.uniform(-6, 6, (20, 1)))).astype(F32)
    y[3] = 0
    q, step = O.quantize_rows_fp8(y)
    dec = O.e4m3_decode(q).astype(np.float64)
    assert step[3] == 0 and not q[3].any()
    for r in range(20):
        if r == 3:
            continue
        assert np.max(np.abs(dec[r])) == 448.0                                       # the row max maps to 448
        t = y[r].astype(np.float64) / np.float64(step[r])
        # round to nearest: the error is at most half the E4M3 spacing at |t| (2^-4 relative, 2^-10 absolute)
        spacing = np.where(np.abs(t) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(t), 1e-300))) - 3))
        assert np.all(np.abs(dec[r] - t) <= spacing / 2 * (1 + 2.0 ** -20) + 1e-12)


def test_gemm_fp8_exact_and_bound():
    rng = np.random.default_rng(8)
    xq = O.e4m3_encode((rng.standard_normal((3, 40)) * 50).astype(F32))
    wq = O.e4m3_encode((rng.standard_normal((4, 40)) * 2).astype(F32))
    acc = O.gemm_fp8(xq, wq)
    xd, wd = O.e4m3_decode(xq), O.e4m3_decode(wq)
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xd[m], wd[n]))
            assert Fraction(float(acc[m, n])) == exact
    # a binary32 accumulation in 128-wide steps stays inside the bound
    big_x = O.e4m3_encode((rng.standard_normal((2, 2048)) * 100).astype(F32))
    big_w = O.e4m3_encode((rng.standard_normal((3, 2048)) * 0.1).astype(F32))
    exact = O.gemm_fp8(big_x, big_w)
    a32 = O.e4m3_decode(big_x).astype(F32)
    b32 = O.e4m3_decode(big_w).astype(F32)
    acc32 = np.zeros((2, 3), F32)
    for k0 in range(0, 2048, 128):
        acc32 = acc32 + (a32[:, k0:k0 + 128] @ b32[:, k0:k0 + 128].T).astype(F32)
    assert np.all(np.abs(acc32 - exact) <= O.gemm_fp8_bound(big_x, big_w))


def test_fold_fp8_and_norm_quant_fp8_reduce_to_the_quantiser():
    rng = np.random.default_rng(2)
    k, n = 128, 9
    a = np.abs(rng.standard_normal(k)).astype(F32) * 4
    w = (rng.standard_normal((n, k)) * 0.02).astype(F32)
    f = O.fold_fp8(a, w, "f32", 0.5)
    q, st = O.quantize_rows_fp8(f["w_hat"])
    assert np.array_equal(f["wq"], q) and np.array_equal(f["w_scale"], st)
    x = rng.standard_normal((4, k)).astype(F32)
    qx, sx, info = O.norm_quant_fp8(x, "f32", "none", f["gamma_f"])
    q2, s2 = O.quantize_rows_fp8(O.normalize(x, "none", gamma=f["gamma_f"]))
    assert np.array_equal(qx, q2) and np.array_equal(sx, s2)
