"""HIP path against the oracle, stage by stage, on seeded inputs (needs an MI355X).

Every stage gets the oracle's own inputs for that stage; codes, steps, smoothing
factors and INT32 accumulators are compared bit for bit, dequantised outputs
within 2e-3 relative (and, the epilogue order being pinned, bit-identical).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import w8a8_int8_linear_amd as sq
from synth import rand_int8, rand_positive, rand_tokens, to_numpy
from tests.gpu_check import check_calibrate, check_fold, check_norm_quant, check_output, host

pytestmark = pytest.mark.gpu
F32 = np.float32
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
OUT_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}


def _seed(*parts):
    return zlib.crc32("/".join(map(str, parts)).encode()) & 0xFFFFF


def cuda(t):
    return None if t is None else t.to("cuda")


def params(k, seed, norm):
    g = torch.Generator().manual_seed(seed)
    gamma = (1 + 0.1 * torch.randn(k, generator=g)).float()
    beta = (0.1 * torch.randn(k, generator=g)).float() if norm == "layernorm" else None
    return gamma, beta


def np_or_none(t):
    return None if t is None else t.numpy()


# --------------------------------------------------------------------------- fused norm + quantise

NQ_SHAPES = [(1, 64), (7, 512), (33, 4096), (5, 9216), (3, 20480), (3, 66560), (2, 81920), (2, 133120)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", NQ_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_norm_quant(dtype, norm, shape):
    m, k = shape
    seed = _seed("nq", dtype, norm, m, k)
    x = rand_tokens(m, k, dtype, seed, n_outliers=max(1, k // 1000), outlier_scale=60.0,
                    mean=0.5 if norm == "layernorm" else 0.0)
    gamma, beta = params(k, seed + 1, norm)
    xq, xs = sq.sq_norm_quant(cuda(x), norm, cuda(gamma), cuda(beta), 1e-5)
    torch.cuda.synchronize()
    check_norm_quant(to_numpy(x), dtype, norm, np_or_none(gamma), np_or_none(beta), 1e-5, host(xq), host(xs),
                     label=f"{dtype}/{norm}/{m}x{k}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_norm_quant_edge_rows(dtype):
    k = 512
    x = torch.zeros(8, k, dtype=torch.float32)
    x[1] = -0.0                                             # signed zeros: step 0, codes 0
    x[2, ::2], x[2, 1::2] = 2.5, -3.5                       # with absmax 127 below the step is exactly 1
    x[2, 0] = 127.0
    x[3] = torch.linspace(-1, 1, k) * 1e-30                 # tiny values
    x[4] = torch.linspace(-1, 1, k) * 3e4                   # large values
    x[5, 17] = -5.0                                          # a single nonzero
    x[6] = 1.0                                               # constant row (LayerNorm variance 0)
    x[7] = torch.arange(k) % 255 - 127                      # every code value
    x = x.to(TORCH_DT[dtype])
    for norm in ["none", "layernorm", "rmsnorm"]:
        xq, xs = sq.sq_norm_quant(cuda(x), norm, None, None, 1e-5)
        torch.cuda.synchronize()
        check_norm_quant(to_numpy(x), dtype, norm, None, None, 1e-5, host(xq), host(xs), label=f"edge/{dtype}/{norm}")
    q = host(sq.sq_norm_quant(cuda(x), "none")[0])
    assert q[2, :4].tolist() == [127, -4, 2, -4] and not q[0].any() and not q[1].any()


def test_norm_quant_near_half_integers():
    """Quotients at and around half-integers, on both sides of the quantiser's 2^-15 residual band:
    y = fl32((n + 1/2 + d) * step) for every n in [-127, 126] and offsets d from 0 to 2^-8, under
    a step of exactly 1 and three steps that are not powers of two. Codes and steps bit for bit."""
    k = 1024
    offs = [0.0] + [s * 2.0 ** e for e in (-22, -18, -16, -15.5, -15, -14.5, -14, -12, -8) for s in (1, -1)]
    rows = []
    for amax in (127.0, 100.0, 3.3e-3, 5.0e4):
        step = np.float32(np.float32(amax) / np.float32(127.0))
        vals = [np.float32((n + 0.5 + d) * np.float64(step)) for d in offs for n in range(-127, 127)]
        row = np.zeros(len(vals) + 1, np.float32)
        row[0] = amax
        row[1:] = np.clip(vals, -amax, amax)
        for start in range(0, row.size, k - 1):
            r = np.zeros(k, np.float32)
            r[0] = amax
            chunk = row[1 + start:1 + start + k - 1]
            r[1:1 + chunk.size] = chunk
            rows.append(r)
    x = torch.from_numpy(np.stack(rows))
    xq, xs = sq.sq_norm_quant(cuda(x), "none", None, None, 1e-5)
    torch.cuda.synchronize()
    check_norm_quant(x.numpy(), "f32", "none", None, None, 1e-5, host(xq), host(xs), label="near-half")
    assert host(xs)[0] == np.float32(1.0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("k", [20480, 66560, 81920])
def test_norm_quant_none_many_rows(dtype, k):
    # many rows per workgroup: the raw-row refill and the per-workgroup column
    # factors (registers / LDS / memory) of every NONE layout
    m = 600
    seed = _seed("nqm", dtype, m, k)
    x = rand_tokens(m, k, dtype, seed, n_outliers=k // 2000, outlier_scale=100.0)
    gamma, _ = params(k, seed + 1, "none")
    xq, xs = sq.sq_norm_quant(cuda(x), "none", cuda(gamma), None, 1e-5)
    torch.cuda.synchronize()
    check_norm_quant(to_numpy(x), dtype, "none", np_or_none(gamma), None, 1e-5, host(xq), host(xs),
                     label=f"{dtype}/none/{m}x{k}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("k", [8192, 16384, 20480])
def test_norm_quant_norms_many_rows(dtype, norm, k):
    # more rows than resident workgroups: each workgroup reuses its on-chip
    # gamma / beta of the first vectors (256 x 4, 512 x 4 and 512 x 5 layouts)
    # over several rows while the next row streams in; every row checked
    m = 600
    seed = _seed("nqn", dtype, norm, m, k)
    x = rand_tokens(m, k, dtype, seed, n_outliers=k // 2000, outlier_scale=60.0)
    gamma, beta = params(k, seed + 1, norm)
    xq, xs = sq.sq_norm_quant(cuda(x), norm, cuda(gamma), cuda(beta), 1e-5)
    torch.cuda.synchronize()
    check_norm_quant(to_numpy(x), dtype, norm, np_or_none(gamma), np_or_none(beta), 1e-5, host(xq), host(xs),
                     label=f"{dtype}/{norm}/{m}x{k}")


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_norm_quant_norms_many_rows_without_params(norm):
    # no gamma / beta: the on-chip copy holds the stand-ins 1 and 0
    m, k = 600, 20480
    x = rand_tokens(m, k, "f16", _seed("nqn0", norm), n_outliers=10, outlier_scale=60.0)
    xq, xs = sq.sq_norm_quant(cuda(x), norm, None, None, 1e-5)
    torch.cuda.synchronize()
    check_norm_quant(to_numpy(x), "f16", norm, None, None, 1e-5, host(xq), host(xs), label=f"noparams/{norm}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_layernorm_mean_offsets(dtype):
    # LayerNorm statistics on both sides of the kernel's switch between the
    # one-pass variance (sum x^2 <= 256 sum (x - mean)^2) and the centred
    # second pass: offsets of 0..1000 spreads, and constant rows
    k = 4096
    g = torch.Generator().manual_seed(77)
    base = torch.randn(12, k, generator=g)
    offsets = torch.tensor([0.0, 1.0, 14.0, 15.0, 15.9, 16.1, 17.0, 40.0, 1000.0, 3.0e3, 0.0, 0.0])
    x = base + offsets[:, None]
    x[10] = 7.25                                             # constant row: variance 0
    x[11] = -3.0e-3                                          # constant, tiny
    x = x.to(TORCH_DT[dtype])
    gamma, beta = params(k, 78, "layernorm")
    xq, xs = sq.sq_norm_quant(cuda(x), "layernorm", cuda(gamma), cuda(beta), 1e-5)
    torch.cuda.synchronize()
    check_norm_quant(to_numpy(x), dtype, "layernorm", np_or_none(gamma), np_or_none(beta), 1e-5, host(xq), host(xs),
                     label=f"offsets/{dtype}")


def test_norm_quant_repeatable():
    x = cuda(rand_tokens(64, 4096, "f16", 5, n_outliers=4))
    g, b = params(4096, 6, "layernorm")
    r1 = sq.sq_norm_quant(x, "layernorm", cuda(g), cuda(b))
    r2 = sq.sq_norm_quant(x, "layernorm", cuda(g), cuda(b))
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


# --------------------------------------------------------------------------- calibration

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", [(1, 64), (5, 4096), (64, 512), (513, 1024), (7, 20480),
                                   # the 1024-thread layouts of 6, 10, 13 and 17 vectors per thread
                                   (5, 40960), (3, 81920), (2, 98304), (3, 133120)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_calibrate(dtype, norm, shape):
    m, k = shape
    seed = _seed("cal", dtype, norm, m, k)
    x = rand_tokens(m, k, dtype, seed, n_outliers=3, outlier_scale=40.0)
    gamma, beta = params(k, seed + 1, norm)
    a = sq.smoothquant_calibrate(cuda(x), norm, cuda(gamma), cuda(beta), 1e-5)
    torch.cuda.synchronize()
    a_ref = check_calibrate(to_numpy(x), dtype, norm, np_or_none(gamma), np_or_none(beta), 1e-5, host(a),
                            label=f"{dtype}/{norm}/{m}x{k}")
    # a second batch keeps the running max
    x2 = rand_tokens(m, k, dtype, seed + 2, n_outliers=3, outlier_scale=40.0)
    sq.smoothquant_calibrate(cuda(x2), norm, cuda(gamma), cuda(beta), 1e-5, absmax=a)
    torch.cuda.synchronize()
    check_calibrate(to_numpy(x2), dtype, norm, np_or_none(gamma), np_or_none(beta), 1e-5, host(a), prior=a_ref,
                    label=f"running/{dtype}/{norm}")


# --------------------------------------------------------------------------- fold

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("alpha", [0.0, 0.5, 0.8, 1.0])
@pytest.mark.parametrize("nk", [(1, 64), (17, 512), (300, 4096)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_fold(dtype, norm, alpha, nk):
    n, k = nk
    seed = _seed("fold", dtype, norm, alpha, n, k)
    w = (rand_tokens(n, k, "f32", seed) * 0.02)
    w[:, 3] = 0.0                                           # a dead input channel hits the eps clamp
    w = w.to(TORCH_DT[dtype])
    act = torch.abs(rand_tokens(1, k, "f32", seed + 1, n_outliers=2, outlier_scale=60.0))[0]
    act[5] = 0.0
    gamma, beta = params(k, seed + 2, norm)
    if norm == "none":
        gamma = beta = None
    out = sq.smoothquant_fold(cuda(act), cuda(w), alpha, 1e-5, norm, cuda(gamma), cuda(beta))
    torch.cuda.synchronize()
    check_fold(act.numpy(), to_numpy(w), dtype, alpha, 1e-5, norm, np_or_none(gamma), np_or_none(beta), out,
               label=f"{dtype}/{norm}/a{alpha}/{n}x{k}")


# --------------------------------------------------------------------------- GEMM

GEMM_SHAPES = [(1, 1, 64), (1, 16, 64), (8, 100, 192), (17, 33, 128), (64, 520, 1024), (65, 64, 64),
               (256, 256, 128), (300, 520, 192), (513, 257, 640), (1000, 1000, 1088), (2, 9216, 9216),
               (600, 700, 4096),
               # decode kernel: every token-tile count, K tails of 64 / 128 / 192 bytes past a 256-byte segment
               (16, 48, 320), (32, 100, 576), (33, 17, 192), (48, 70, 4160), (63, 130, 2112), (64, 2048, 9216),
               (5, 36, 1984),
               # decode kernel, 9-tile strips (N >= 16384) of N / CUs channels rounded up to a multiple of 4
               # (68 at N = 16400 and 16416, 64 at 16384, 116 at 28700, 80 at 20000): ragged last strips,
               # K tails
               (33, 16400, 320), (20, 16384, 1088), (64, 16416, 2112), (12, 16400, 704), (9, 300, 1216),
               (40, 28700, 320), (7, 20000, 192),
               # eight token tiles (65-128 tokens) on both strip widths, K tails; 129 takes the prefill tile
               (100, 9216, 9216), (128, 36864, 2112), (77, 16400, 1216), (129, 520, 640),
               # up to 4 tokens: the MFMA decode kernel below N = 16384, the GEMV from there; K tails inside a
               # 256-byte segment, ragged N
               (3, 130, 320), (4, 16400, 1216), (2, 77, 704), (1, 1000, 4160),
               (1, 16400, 4160), (2, 16390, 704), (3, 20000, 320), (4, 16384, 64),
               # 1-2 tokens: the row GEMV up to K = 9216 (ragged N, K not a multiple of 1024), past it the
               # GEMV (N >= 16384) or the MFMA decode kernel; row counts that leave a last, partial round
               # of rows over the 2048 waves (9216, 4099, 5000, 2100, 3072)
               (1, 9217, 9216), (2, 4099, 4160), (1, 5, 64), (2, 300, 9152), (1, 9216, 9216), (1, 5000, 1088),
               (2, 2100, 9216), (1, 3072, 4096),
               (1, 16400, 20480), (2, 3000, 13312)]


@pytest.mark.parametrize("mnk", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_i32_exact(mnk):
    m, n, k = mnk
    xq = rand_int8((m, k), 100 + m)
    wq = rand_int8((n, k), 200 + n)
    acc = sq.sq_w8a8_gemm(cuda(xq), None, cuda(wq), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    ref = O.int_gemm(xq.numpy(), wq.numpy())
    got = host(acc).astype(np.int64)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} accumulators differ"



# The decode kernel picks its wave grid (token groups x channel groups) from the token-tile count and
# the strip width: every token count up to 64 and a spread of 65-128 (eight token tiles), on a ragged
# narrow strip (the MFMA kernel throughout) and on the 9-tile strips (the GEMV up to 4 tokens),
# with an odd number of 64-byte K steps (the last segment's second half is the next row's bytes).
DECODE_MS = list(range(1, 65)) + [65, 72, 80, 96, 111, 112, 127, 128]


# A decode workgroup takes N / CUs channels rounded up to a multiple of 4, in 3 tiles below N = 16384
# (4 at N = 300, 40 at N = 9250 with a 10-row last strip) and 9 tiles from there (68 at N = 16400,
# a 12-row last strip).
@pytest.mark.parametrize("m", DECODE_MS)
@pytest.mark.parametrize("nk", [(300, 192), (9250, 256), (16400, 320)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_decode_every_token_count(m, nk):
    n, k = nk
    xq = rand_int8((m, k), 300 + m)
    wq = rand_int8((n, k), 400 + n)
    acc = sq.sq_w8a8_gemm(cuda(xq), None, cuda(wq), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    ref = O.int_gemm(xq.numpy(), wq.numpy())
    got = host(acc).astype(np.int64)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} accumulators differ"



# More tiles than resident workgroups: the prefill kernel's workgroups loop over several tiles (each
# tile's epilogue overlapping the next tile's first stages), with ragged last tile-rows and -columns.
# Every tile-row is sampled (every 16th row and the edges) against all columns.
# The launch picks the tile width (256, 192 or 128 columns) whose grid wastes least of its last wave:
# 2100 x 8000, 4097 x 16385 and 257 x 33000 take 192-column tiles, 1281 x 10760 and 513 x 32648
# 128-column ones (2 and 3 tiles per workgroup), the rest 256.
PERSIST_SHAPES = [(2100, 8000, 256), (4097, 16385, 128), (1100, 30000, 384), (257, 33000, 256), (1281, 10760, 256),
                  (513, 32648, 128)]


def _persist_rows(m):
    return np.unique(np.r_[np.arange(0, m, 16), [255, 256, m - 2, m - 1]])


@pytest.mark.parametrize("mnk", PERSIST_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_persistent_grid_accumulators(mnk):
    m, n, k = mnk
    xq, wq = rand_int8((m, k), 800 + m), rand_int8((n, k), 900 + n)
    acc = sq.sq_w8a8_gemm(cuda(xq), None, cuda(wq), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = _persist_rows(m)
    ref = O.int_gemm(xq.numpy()[rows], wq.numpy())
    got = host(acc)[rows].astype(np.int64)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} accumulators differ"


# Seeded random prefill shapes: every tile width (the launch picks 256, 192 or 128 columns from the
# grid), both stage kernels (K % 128 == 0 and 64), ragged edges, one to several tiles per workgroup.
# One random row per 256-row tile-row and the edge rows, against all columns.
def _random_gemm_shapes(count=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        m, n, k = int(rng.integers(65, 3000)), int(rng.integers(1, 24000)), int(rng.integers(1, 48)) * 64
        if m * n * k <= 6e10:
            out.append((m, n, k))
    return out


@pytest.mark.parametrize("mnk", _random_gemm_shapes(), ids=lambda s: "x".join(map(str, s)))
def test_gemm_random_prefill_shapes(mnk):
    m, n, k = mnk
    xq, wq = rand_int8((m, k), 1000 + m), rand_int8((n, k), 2000 + n)
    acc = sq.sq_w8a8_gemm(cuda(xq), None, cuda(wq), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(m * n + k)
    rows = np.unique(np.r_[np.minimum(np.arange(0, m, 256) + rng.integers(0, 256, -(-m // 256)), m - 1), [0, m - 1]])
    ref = O.int_gemm(xq.numpy()[rows], wq.numpy())
    got = host(acc)[rows].astype(np.int64)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} accumulators differ"


@pytest.mark.parametrize("out", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mnk", [(2100, 8000, 256), (1281, 10760, 256)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_persistent_grid_dequant_with_bias(out, mnk):
    m, n, k = mnk
    xq, wq = rand_int8((m, k), 810), rand_int8((n, k), 910)
    xs, ws = rand_positive(m, 820, 1e-3, 0.5), rand_positive(n, 920, 1e-4, 0.05)
    b = rand_tokens(1, n, "f32", 930)[0]
    y = sq.sq_w8a8_gemm(cuda(xq), cuda(xs), cuda(wq), cuda(ws), cuda(b), out_dtype=OUT_DT[out])
    torch.cuda.synchronize()
    rows = _persist_rows(m)
    acc = O.int_gemm(xq.numpy()[rows], wq.numpy())
    out_ref, v32 = O.dequantize(acc, xs.numpy()[rows], ws.numpy(), b.numpy(), out)
    check_output(host(y)[rows], out_ref, v32, out, label=f"{out}/{m}x{n}x{k}")

def test_gemm_int32_range_at_max_k():
    k = sq.SQ_K_MAX
    for m in [3, 70]:                                        # GEMV and tiled kernels
        xq = torch.full((m, k), 127, dtype=torch.int8)
        xq[1] = -127
        wq = torch.full((5, k), 127, dtype=torch.int8)
        wq[2] = -127
        acc = host(sq.sq_w8a8_gemm(cuda(xq), None, cuda(wq), None, out_dtype=torch.int32)).astype(np.int64)
        assert np.array_equal(acc, O.int_gemm(xq.numpy(), wq.numpy()))
        assert acc.max() == k * 127 * 127


def test_gemm_minus_128_codes_up_to_their_k_limit():
    # -128 is a legal int8 operand although no quantiser here produces it: the products are exact, and
    # the sum stays inside int32 while K * 128^2 < 2^31, i.e. up to K = 131008 (a multiple of 64)
    k = 131008
    assert k * 128 * 128 < 2 ** 31 <= (k + 64) * 128 * 128
    for m, n in [(3, 5), (40, 300), (70, 5), (300, 520)]:     # decode and tiled kernels, K % 128 == 64
        xq = torch.full((m, k), -128, dtype=torch.int8)
        xq[1] = 127
        wq = torch.full((n, k), -128, dtype=torch.int8)
        wq[2] = 127
        wq[3, ::2] = 0
        acc = host(sq.sq_w8a8_gemm(cuda(xq), None, cuda(wq), None, out_dtype=torch.int32)).astype(np.int64)
        assert np.array_equal(acc, O.int_gemm(xq.numpy(), wq.numpy())), f"{m}x{n}"
        assert acc.max() == k * 128 * 128 and acc.min() == -k * 128 * 127


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bias", [False, True])
# 16-bit outputs of the tiled kernels go out 8 columns per lane when N % 8 == 0 (ragged last tile
# included), element by element otherwise; K % 128 == 64 takes the 64-byte kernel. The decode paths
# have epilogues of their own: the row GEMV (1 x 72), the wide GEMV (up to 4 tokens from N = 16384,
# N % 4 both ways), 3-tile and 9-tile strips (40 tokens) and eight token tiles (100 tokens).
@pytest.mark.parametrize("mnk", [(1, 72, 64), (40, 300, 512), (300, 520, 192), (777, 1030, 1024),
                                 (777, 1032, 1024), (300, 776, 192), (257, 1028, 256),
                                 (3, 16400, 128), (2, 16390, 64), (40, 16402, 192), (100, 522, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_dequant(out, bias, mnk):
    m, n, k = mnk
    xq, wq = rand_int8((m, k), 300 + m), rand_int8((n, k), 400 + n)
    xs, ws = rand_positive(m, 500 + m, 1e-3, 0.5), rand_positive(n, 600 + n, 1e-4, 0.05)
    b = (rand_tokens(1, n, "f32", 700 + n)[0]) if bias else None
    y = sq.sq_w8a8_gemm(cuda(xq), cuda(xs), cuda(wq), cuda(ws), cuda(b), out_dtype=OUT_DT[out])
    torch.cuda.synchronize()
    acc = O.int_gemm(xq.numpy(), wq.numpy())
    out_ref, v32 = O.dequantize(acc, xs.numpy(), ws.numpy(), None if b is None else b.numpy(), out)
    check_output(host(y), out_ref, v32, out, label=f"{out}/{m}x{n}x{k}")
