"""FP8 (OCP E4M3) variant on the HIP path against the oracle (needs an MI355X). Quantiser and
fold codes and steps bit for bit; the GEMM against the oracle's exact sum within the error of
the matrix cores' FP8 summation.

That summation is not a plain binary32 accumulation. Measured with crafted inputs (and pinned
by test_fp8_mfma_group_truncation below), v_mfma_scale_f32_16x16x128_f8f6f4 sums the products
of each group of 8 consecutive K positions in a fixed-point window whose lowest bit is
2^(E - 13), E the largest sum of the two operands' unbiased exponents in the group; every
product is truncated toward zero to that window; the group sums then reach the binary32
accumulator. So |acc - exact| <= sum_k (|p_k| mod 2^(E_g - 13)) + (K/8 + 3) 2^-24 sum_k |p_k|,
the second term bounding every binary32 rounding of group sums and partial sums in any order.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import w8a8_int8_linear_amd as sq
from synth import rand_tokens, site_inputs, to_numpy
from tests.fp8_model import fp8_gemm_tolerance, fp8_mfma_model
from tests.gpu_check import bits, check_calibrate, host

pytestmark = pytest.mark.gpu
F32 = np.float32


def _seed(*parts):
    return zlib.crc32("/".join(map(str, parts)).encode()) & 0xFFFFF


def _cuda(t):
    return None if t is None else t.to("cuda")


def _np(t):
    return None if t is None else t.numpy()


def check_nq_fp8(x_np, dtype, norm, g, b, eps, xq_gpu, xs_gpu, label):
    q, step, info = O.norm_quant_fp8(x_np, dtype, norm, g, b, eps)
    bad = np.where((q != xq_gpu).any(axis=1) | (bits(step) != bits(xs_gpu)))[0]
    for r in bad:
        assert info["near_tie"][r], f"{label}: row {r} differs ({int((q[r] != xq_gpu[r]).sum())} codes)"
        st = O.row_stats(O.widen(x_np[r:r + 1], dtype)[0], norm)
        ok = False
        for mu in {float(st["mu"]), float(st["mu_other"])}:
            for var in {float(st["var"]), float(st["var_other"])}:
                y = O.normalize(O.widen(x_np[r:r + 1], dtype), norm, [mu], [var], g, b, eps)
                vq, vs = O.quantize_rows_fp8(y)
                ok |= np.array_equal(vq[0], xq_gpu[r]) and bits(vs)[0] == bits(xs_gpu[r:r + 1])[0]
        assert ok, f"{label}: near-tie row {r} matches no correct rounding"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", [(1, 64), (7, 512), (33, 4096), (3, 20480), (2, 81920), (2, 133120)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_norm_quant_fp8(dtype, norm, shape):
    m, k = shape
    seed = _seed("nq8", dtype, norm, m, k)
    x = rand_tokens(m, k, dtype, seed, n_outliers=max(1, k // 1000), outlier_scale=60.0,
                    mean=0.5 if norm == "layernorm" else 0.0)
    g = torch.Generator().manual_seed(seed + 1)
    gamma = (1 + 0.1 * torch.randn(k, generator=g)).float()
    beta = (0.1 * torch.randn(k, generator=g)).float() if norm == "layernorm" else None
    xq, xs = sq.sq_norm_quant_fp8(_cuda(x), norm, _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    check_nq_fp8(to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5, host(xq), host(xs), f"{dtype}/{norm}/{m}x{k}")


def test_norm_quant_fp8_edge_rows():
    # zeros, tiny values in E4M3's subnormal range, exact midpoints of the E4M3 grid, a huge outlier
    k = 512
    x = np.zeros((6, k), F32)
    x[1] = np.linspace(-448, 448, k).astype(F32)
    x[2, :] = 1e-3
    x[2, 0] = 448.0                                    # others land in E4M3's subnormal range
    mids = (O.e4m3_decode(np.arange(1, 0x7E, dtype=np.uint8)).astype(np.float64)
            + O.e4m3_decode(np.arange(2, 0x7F, dtype=np.uint8)).astype(np.float64)) / 2
    x[3, :len(mids)] = mids.astype(F32)
    x[3, -1] = 448.0                                   # step exactly 1: every midpoint is a tie
    x[4] = np.random.default_rng(1).standard_normal(k).astype(F32)
    x[4, 7] = 3e4
    x[5, ::2] = -0.0
    xq, xs = sq.sq_norm_quant_fp8(torch.from_numpy(x).cuda(), "none")
    torch.cuda.synchronize()
    q, st, _ = O.norm_quant_fp8(x, "f32", "none")
    assert np.array_equal(bits(st), bits(host(xs)))
    assert np.array_equal(q, host(xq))


def check_fold_fp8(a_ref, w_np, dtype, alpha, eps, norm, gamma, beta, out_gpu, label=""):
    """s (either rounding at a near-tie), gamma', beta', E4M3 codes and steps of every W row bit for bit."""
    s_ref, dist, other = O.smoothing_factors(a_ref, O.weight_colmax(w_np, dtype), alpha, eps)
    s_gpu = host(out_gpu["s"])
    diff = bits(s_ref) != bits(s_gpu)
    ok = (dist < O.smoothquant_oracle.NEAR_TIE) & (bits(other) == bits(s_gpu))
    assert ok[diff].all(), f"{label}: s differs at {np.where(diff & ~ok)[0][:8]}"
    f = O.fold_fp8(a_ref, w_np, dtype, alpha, eps, norm, gamma, beta, s=np.where(diff, other, s_ref))
    assert np.array_equal(bits(f["gamma_f"]), bits(host(out_gpu["gamma_f"]))), f"{label}: gamma' differs"
    if f["beta_f"] is not None:
        assert np.array_equal(bits(f["beta_f"]), bits(host(out_gpu["beta_f"]))), f"{label}: beta' differs"
    bad = np.where((f["wq"] != host(out_gpu["wq"])).any(axis=1))[0]
    assert not len(bad), f"{label}: weight codes differ in rows {bad[:8]}"
    assert np.array_equal(bits(f["w_scale"]), bits(host(out_gpu["w_scale"]))), f"{label}: w_scale differs"
    return f


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm"])
@pytest.mark.parametrize("nk", [(48, 512), (300, 4096), (64, 81920)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_fold_fp8(dtype, norm, nk):
    n, k = nk
    seed = _seed("fold8", dtype, norm, n, k)
    g = torch.Generator().manual_seed(seed)
    a = (torch.rand(k, generator=g) * 5 + 0.01).float()
    a[:: max(1, k // 7)] *= 40.0
    w = (torch.randn(n, k, generator=g) * 0.02).to({"f32": torch.float32, "f16": torch.float16,
                                                     "bf16": torch.bfloat16}[dtype])
    gamma = (1 + 0.1 * torch.randn(k, generator=g)).float() if norm != "none" else None
    beta = (0.1 * torch.randn(k, generator=g)).float() if norm == "layernorm" else None
    out = sq.smoothquant_fold_fp8(_cuda(a), _cuda(w), 0.5, 1e-5, norm, _cuda(gamma), _cuda(beta))
    torch.cuda.synchronize()
    check_fold_fp8(a.numpy(), to_numpy(w), dtype, 0.5, 1e-5, norm, _np(gamma), _np(beta), out,
                   f"{dtype}/{norm}/{n}x{k}")


def _codes(shape, seed, scale):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal(shape) * scale).astype(F32)
    v = np.clip(v, -448, 448)
    return O.e4m3_encode(v)


def _positions(m, n, k, seed, full_limit=6e7, samples=3000):
    if m * n * k <= full_limit:
        mm, nn = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        return mm.ravel(), nn.ravel()
    rng = np.random.default_rng(seed)
    mi = np.concatenate([rng.integers(0, m, samples), [0, m - 1, m - 1, 0]])
    ni = np.concatenate([rng.integers(0, n, samples), [0, n - 1, 0, n - 1]])
    return mi, ni


def test_fp8_mfma_group_truncation():
    """The summation model's predictions on crafted cases, exactly: which K positions share a group,
    truncation toward zero for either sign, and the window set by the operands' exponent sum."""
    k = 128
    xs, ws = [], []

    def case(pairs, k=k):
        x, w = np.zeros(k, F32), np.ones(k, F32)
        for pos, xv, wv in pairs:
            x[pos], w[pos] = xv, wv
        xs.append(x)
        ws.append(w)

    for b in (0, 21, 72, 120):
        for j in range(b - 9, b + 10):
            if 0 <= j < k and j != b:
                case([(b, 256.0, 1.0), (j, 2.0 ** -6, 1.0)])
    for c in (1.25, 1.5, 1.875, 2.25, 3.75):
        for sgn in (1.0, -1.0):
            case([(0, 256.0, 1.0), (1, sgn * c * 2.0 ** -6, 1.0)])
            case([(0, -256.0, 1.0), (1, sgn * c * 2.0 ** -6, 1.0)])
    for t in range(0, 7):
        case([(0, 448.0, 448.0), (1, 2.0 ** t, 1.0)])
    for t in range(4, 9):
        case([(0, 240.0, 1.0), (1, 2.0 ** -t, 1.0)])
        case([(0, 15.0, 15.0), (1, 2.0 ** -t, 1.0)])
    for t in range(0, 12):
        case([(0, 256.0, 1.0), (64 + 8 * (t % 4) + 1, 2.0 ** -min(t, 9), 1.0), (3, 2.0 ** -9, 1.0)])
    xq, wq = O.e4m3_encode(np.array(xs)), O.e4m3_encode(np.array(ws))
    assert np.array_equal(O.e4m3_decode(xq), np.array(xs)) and np.array_equal(O.e4m3_decode(wq), np.array(ws))
    want = fp8_mfma_model(xq, wq)
    assert not np.array_equal(want, O.gemm_fp8(xq, wq).diagonal())    # the cases do exercise truncation
    got = np.empty(len(xs))
    for a in range(0, len(xs), 64):
        xb, wb = xq[a:a + 64], wq[a:a + 64]
        y = sq.sq_fp8_gemm(torch.from_numpy(xb).cuda(), torch.ones(len(xb), device="cuda"),
                           torch.from_numpy(wb).cuda(), torch.ones(len(wb), device="cuda"), out_dtype=torch.float32)
        got[a:a + 64] = host(y).astype(np.float64).diagonal()
    bad = np.where(got != want)[0]
    assert not len(bad), f"cases {bad[:8]}: gpu {got[bad[:4]]} model {want[bad[:4]]}"


GEMM_SHAPES = [(17, 33, 128), (256, 256, 128), (300, 520, 384), (513, 700, 1280), (64, 16416, 2176),
               (1024, 2048, 20480), (5, 9, 133120),
               # decode (M <= 128): every token-tile count, 3-tile and 9-tile strips, ragged N
               (1, 9216, 9216), (2, 1000, 1280), (4, 36864, 9216), (16, 130, 384), (33, 4000, 2048),
               (48, 16400, 1024), (64, 36864, 9216), (65, 300, 256), (128, 36864, 2048), (129, 300, 256),
               # N not a multiple of 4: the epilogue's partial stores, prefill and decode
               (130, 45, 256), (300, 1001, 384), (40, 37, 640)]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_gemm_accumulator(shape):
    m, n, k = shape
    xq = _codes((m, k), m + n, 40.0)
    wq = _codes((n, k), m * n + 1, 0.5)
    ones_m, ones_n = torch.ones(m, device="cuda"), torch.ones(n, device="cuda")
    y = sq.sq_fp8_gemm(torch.from_numpy(xq).cuda(), ones_m, torch.from_numpy(wq).cuda(), ones_n,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    mi, ni = _positions(m, n, k, m * n)
    exact, tol = fp8_gemm_tolerance(xq, wq, mi, ni)
    if len(mi) == m * n:
        assert np.array_equal(exact, O.gemm_fp8(xq, wq).ravel())        # same sums as the oracle's matmul
    err = np.abs(host(y)[mi, ni].astype(np.float64) - exact)
    assert np.all(err <= tol), f"max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3g}"


# Every token count the FP8 decode kernel serves up to 64 and a spread of 65-128 (eight token tiles),
# and so every wave grid it picks, on narrow strips (4 channels at N = 300; 40 at N = 9250, the last
# strip 10 rows) and on 9-tile strips (68 channels at N = 16400), three 128-byte segments.
@pytest.mark.parametrize("m", list(range(1, 65)) + [65, 80, 96, 127, 128])
@pytest.mark.parametrize("n", [300, 9250, 16400])
def test_fp8_gemm_decode_every_token_count(m, n):
    k = 384
    xq = _codes((m, k), 500 + m, 40.0)
    wq = _codes((n, k), 600 + n, 0.5)
    ones_m, ones_n = torch.ones(m, device="cuda"), torch.ones(n, device="cuda")
    y = sq.sq_fp8_gemm(torch.from_numpy(xq).cuda(), ones_m, torch.from_numpy(wq).cuda(), ones_n,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    mi, ni = _positions(m, n, k, m * n)
    exact, tol = fp8_gemm_tolerance(xq, wq, mi, ni)
    err = np.abs(host(y)[mi, ni].astype(np.float64) - exact)
    assert np.all(err <= tol), f"max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3g}"


# More tiles than resident workgroups: the FP8 prefill kernel's workgroups loop over several tiles,
# with ragged last tile-rows and -columns; sampled positions cover every 256 x 128 region (the
# narrowest tile). 2100 x 8000 takes 192-column tiles, 1281 x 10760 128-column ones (two per
# workgroup), 4097 x 9000 256-column ones.
@pytest.mark.parametrize("shape", [(2100, 8000, 256), (4097, 9000, 384), (1281, 10760, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_gemm_persistent_grid(shape):
    m, n, k = shape
    xq = _codes((m, k), 11 + m, 40.0)
    wq = _codes((n, k), 13 + n, 0.5)
    rng = np.random.default_rng(m + n)
    xs = (rng.uniform(0.5, 2, m) * 1e-2).astype(F32)
    ws = (rng.uniform(0.5, 2, n) * 1e-3).astype(F32)
    bias = rng.standard_normal(n).astype(F32)
    y = sq.sq_fp8_gemm(torch.from_numpy(xq).cuda(), torch.from_numpy(xs).cuda(), torch.from_numpy(wq).cuda(),
                       torch.from_numpy(ws).cuda(), torch.from_numpy(bias).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    tm, tn = np.meshgrid(np.arange(-(-m // 256)), np.arange(-(-n // 128)), indexing="ij")
    mi = np.concatenate([np.minimum(tm.ravel() * 256 + rng.integers(0, 256, tm.size), m - 1),
                         rng.integers(0, m, 2000), [0, m - 1, m - 1, 0]])
    ni = np.concatenate([np.minimum(tn.ravel() * 128 + rng.integers(0, 128, tn.size), n - 1),
                         rng.integers(0, n, 2000), [0, n - 1, 0, n - 1]])
    acc, tol_acc = fp8_gemm_tolerance(xq, wq, mi, ni)
    scale = xs.astype(np.float64)[mi] * ws.astype(np.float64)[ni]
    b = bias.astype(np.float64)[ni]
    ref = acc * scale + b
    tol = (tol_acc * scale * (1 + 2.0 ** -20) + ((np.abs(acc) + tol_acc) * scale + np.abs(b)) * 3 * 2.0 ** -24
           + np.abs(ref) * 2.0 ** -24 + 2.0 ** -24)
    err = np.abs(host(y)[mi, ni].astype(np.float64) - ref)
    assert np.all(err <= tol), f"max excess {np.max(err - tol):.3g}"


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
# prefill tiles, then the decode kernel's FP8 mode: one token, 3-tile strips, 9-tile strips (N % 4 != 0)
# and eight token tiles
@pytest.mark.parametrize("mnk", [(300, 520, 1280), (257, 1030, 384), (1, 72, 128), (40, 1000, 256),
                                 (8, 16402, 128), (100, 522, 256)], ids=lambda s: "x".join(map(str, s)))
def test_fp8_gemm_dequantised_output(out, mnk):
    m, n, k = mnk
    xq = _codes((m, k), 5, 30.0)
    wq = _codes((n, k), 6, 1.0)
    rng = np.random.default_rng(7)
    xs = (rng.uniform(0.5, 2, m) * 1e-2).astype(F32)
    ws = (rng.uniform(0.5, 2, n) * 1e-3).astype(F32)
    bias = rng.standard_normal(n).astype(F32) if out != "bf16" else None
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out]
    y = sq.sq_fp8_gemm(torch.from_numpy(xq).cuda(), torch.from_numpy(xs).cuda(), torch.from_numpy(wq).cuda(),
                       torch.from_numpy(ws).cuda(), None if bias is None else torch.from_numpy(bias).cuda(),
                       out_dtype=dt)
    torch.cuda.synchronize()
    mi, ni = _positions(m, n, k, 11)
    acc, tol_acc = fp8_gemm_tolerance(xq, wq, mi, ni)
    scale = xs.astype(np.float64)[mi] * ws.astype(np.float64)[ni]
    b = 0 if bias is None else bias.astype(np.float64)[ni]
    ref = acc * scale + b
    yg = y.float().cpu().numpy()[mi, ni].astype(np.float64)
    out_u = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[out]
    # the accumulator's tolerance carried through the scales, the epilogue's binary32 roundings (relative
    # to the scaled accumulator and the bias), then one rounding to the output type
    tol = (tol_acc * scale * (1 + 2.0 ** -20) + ((np.abs(acc) + tol_acc) * scale + np.abs(b)) * 3 * 2.0 ** -24
           + np.abs(ref) * out_u + 2.0 ** -24)
    assert np.all(np.abs(yg - ref) <= tol), f"max excess {np.max(np.abs(yg - ref) - tol):.3g}"


def test_fp8_layer_end_to_end():
    """calibrate -> FP8 fold -> FP8 norm+quantise -> FP8 GEMM on a prefill site, stage by stage."""
    inp = site_inputs(2, 0, m=256, device="cuda")
    x, xc, w, g, b = inp["x"], inp["x_cal"], inp["w"], inp["gamma"], inp["beta"]
    amax = sq.smoothquant_calibrate(xc, "layernorm", g, b, 1e-5)
    fo = sq.smoothquant_fold_fp8(amax, w, 0.5, 1e-5, "layernorm", g, b)
    xq, xs = sq.sq_norm_quant_fp8(x, "layernorm", fo["gamma_f"], fo["beta_f"], 1e-5)
    y = sq.sq_fp8_gemm(xq, xs, fo["wq"], fo["w_scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_calibrate(to_numpy(xc), "f16", "layernorm", host(g), host(b), 1e-5, host(amax), label="e2e calibrate")
    f = check_fold_fp8(host(amax), to_numpy(w), "f16", 0.5, 1e-5, "layernorm", host(g), host(b), fo, "e2e fold")
    check_nq_fp8(to_numpy(x), "f16", "layernorm", f["gamma_f"], f["beta_f"], 1e-5, host(xq), host(xs), "e2e")
    q = host(xq)
    m, n = q.shape[0], f["wq"].shape[0]
    mi, ni = _positions(m, n, q.shape[1], 3)
    acc, tol_acc = fp8_gemm_tolerance(q, f["wq"], mi, ni)
    scale = host(xs).astype(np.float64)[mi] * f["w_scale"].astype(np.float64)[ni]
    ref = acc * scale
    err = np.abs(host(y)[mi, ni].astype(np.float64) - ref)
    assert np.all(err <= tol_acc * scale * (1 + 2.0 ** -20) + (np.abs(acc) + tol_acc) * scale * 3 * 2.0 ** -24 + 1e-30)
