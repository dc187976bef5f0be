"""Per-tensor granularities on the HIP path against the oracle (needs an MI355X): one dynamic
step for the whole activation tensor, a static calibrated step with clipping, the static step
itself, and the fold with one weight step. Codes, steps and outputs bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
import w8a8_int8_linear_amd as sq
from synth import rand_tokens, to_numpy
from tests.gpu_check import bits, check_calibrate, host

pytestmark = pytest.mark.gpu
F32 = np.float32
SHAPES = [(1, 64), (7, 512), (33, 4096), (3000, 512), (5, 9216), (3, 20480), (2, 81920), (2, 133120)]


def _seed(*parts):
    return zlib.crc32("/".join(map(str, parts)).encode()) & 0xFFFFF


def _params(k, seed, norm):
    g = torch.Generator().manual_seed(seed)
    gamma = (1 + 0.1 * torch.randn(k, generator=g)).float()
    beta = (0.1 * torch.randn(k, generator=g)).float() if norm == "layernorm" else None
    return gamma, beta


def _cuda(t):
    return None if t is None else t.to("cuda")


def _np(t):
    return None if t is None else t.numpy()


def _inputs(tag, dtype, norm, m, k):
    seed = _seed(tag, dtype, norm, m, k)
    x = rand_tokens(m, k, dtype, seed, n_outliers=max(1, k // 1000), outlier_scale=60.0,
                    mean=0.5 if norm == "layernorm" else 0.0)
    gamma, beta = _params(k, seed + 1, norm)
    return x, gamma, beta


def _compare(q_ref, xs_ref, info, xq_gpu, xs_gpu, label, src, fp8=False):
    """Steps bit for bit; codes bit for bit, except on a row whose statistics are a near-tie, whose
    codes must then be those of one of the row's correct roundings (the oracle's candidate y rows,
    quantised with the same step for the whole tensor). src = (x, dtype, norm, gamma_f, beta_f, eps)."""
    tie = info["near_tie"]
    assert np.array_equal(bits(xs_ref), bits(xs_gpu)), f"{label}: step {xs_ref[0]!r} vs {xs_gpu[0]!r}"
    bad = np.where((q_ref != xq_gpu).any(axis=1))[0]
    assert all(tie[r] for r in bad), f"{label}: rows {bad[:8]} differ"
    x_np, dtype, norm, gamma_f, beta_f, eps = src
    quant = O.quantize_tensor_fp8 if fp8 else O.quantize_tensor
    for r in bad:
        cands = [quant(y, step=xs_ref[0])[0][0] for y in O.row_y_variants(x_np[r], dtype, norm, gamma_f, beta_f, eps)]
        assert any(np.array_equal(c, xq_gpu[r]) for c in cands), f"{label}: near-tie row {r} matches no rounding"
    return len(bad)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_norm_quant_per_tensor(dtype, norm, shape):
    m, k = shape
    x, gamma, beta = _inputs("nqt", dtype, norm, m, k)
    xq, xs = sq.sq_norm_quant_per_tensor(_cuda(x), norm, _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    q, xsr, info = O.norm_quant_per_tensor(to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5)
    _compare(q, xsr, info, host(xq), host(xs), f"{dtype}/{norm}/{m}x{k}",
             (to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", [(7, 512), (33, 4096), (3, 20480), (2, 81920)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("factor", [0.37, 1.0, 2.5])
def test_norm_quant_static(dtype, norm, shape, factor):
    # factor < 1: a step below the tensor's own, so the largest values clip
    m, k = shape
    x, gamma, beta = _inputs("nqs", dtype, norm, m, k)
    _, xs_dyn, _ = O.norm_quant_per_tensor(to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5)
    step = F32(xs_dyn[0] * F32(factor))
    st = torch.tensor([step], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_static(_cuda(x), st, norm, _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    q, xsr, info = O.norm_quant_per_tensor(to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5, step=step)
    _compare(q, xsr, info, host(xq), host(xs), f"{dtype}/{norm}/{m}x{k}/x{factor}",
             (to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5))
    if factor < 1:
        assert (np.abs(host(xq).astype(np.int32)) == 127).sum() > 1       # clipping happened


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("factor", [1e-5, 1e-20, 2.0 ** -120])
def test_norm_quant_static_far_below_range(dtype, factor):
    """Static steps far below the tensor's own: quotients from the clipping edge up to far past
    2^22 (the fast path's magic-constant range), and (2^-120) steps below 2^-100, which always
    divide. Codes and steps bit for bit against the oracle."""
    m, k = 33, 4096
    x, gamma, beta = _inputs("nqf", dtype, "layernorm", m, k)
    _, xs_dyn, _ = O.norm_quant_per_tensor(to_numpy(x), dtype, "layernorm", _np(gamma), _np(beta), 1e-5)
    step = F32(np.float64(xs_dyn[0]) * factor)
    assert step > 0
    st = torch.tensor([step], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_static(_cuda(x), st, "layernorm", _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):
        q, xsr, info = O.norm_quant_per_tensor(to_numpy(x), dtype, "layernorm", _np(gamma), _np(beta), 1e-5, step=step)
    _compare(q, xsr, info, host(xq), host(xs), f"{dtype}/x{factor}",
             (to_numpy(x), dtype, "layernorm", _np(gamma), _np(beta), 1e-5))
    assert (np.abs(host(xq).astype(np.int32)) == 127).mean() > 0.9


def test_norm_quant_static_product_overflow():
    """binary32 values near 1e30 with a static step of 1e-12: y times the reciprocal of the step overflows binary32,
    which must send those elements to the divide path (codes +-127, sign kept)."""
    g = torch.Generator().manual_seed(7)
    x = (torch.randn(5, 1024, generator=g) * 1e30).float()
    x[0, :8] = torch.tensor([0.0, -0.0, 1e-30, -1e-30, 3e-12, -3e-12, 1e-12, 5e-13])
    step = F32(1e-12)
    st = torch.tensor([step], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_static(_cuda(x), st, "none")
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):                     # the oracle's quotients overflow to inf, then clip
        q, xsr, info = O.norm_quant_per_tensor(x.numpy(), "f32", "none", None, None, 1e-5, step=step)
    assert np.array_equal(q, host(xq)) and np.array_equal(bits(xsr), bits(host(xs)))
    assert set(np.unique(q[:, 8:])) <= {-127, 127}


@pytest.mark.parametrize("step", [1.5 * 2.0 ** 126, 3.0e38])
def test_norm_quant_static_huge_step(step):
    """A static step above 2^126, where fl32(1/step) is subnormal: quotients of binary32 values up to
    FLT_MAX stay below 4, and half-integer quotients must still round to even."""
    g = torch.Generator().manual_seed(11)
    x = (torch.rand(6, 512, generator=g) * 2 - 1).double() * 3.4e38
    st32 = np.float32(step)
    halves = [k for k in (0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 1.0, -1.0) if abs(k) * float(st32) < 3.4e38]
    x[0, :len(halves)] = torch.tensor(halves, dtype=torch.float64) * float(st32)   # exact in binary32
    x = x.float()
    assert torch.isfinite(x).all()
    st = torch.tensor([st32], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_static(_cuda(x), st, "none")
    torch.cuda.synchronize()
    q, xsr, info = O.norm_quant_per_tensor(x.numpy(), "f32", "none", None, None, 1e-5, step=st32)
    assert np.array_equal(q, host(xq)) and np.array_equal(bits(xsr), bits(host(xs)))
    assert q[0, :len(halves)].tolist() == [int(np.rint(k)) for k in halves]


@pytest.mark.parametrize("step", [0.0, -1.0])
def test_norm_quant_static_nonpositive_step_gives_zero_codes(step):
    x, gamma, beta = _inputs("nqz", "f16", "layernorm", 9, 4096)
    st = torch.tensor([step], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_static(_cuda(x), st, "layernorm", _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    assert not host(xq).any()
    assert (host(xs) == F32(step)).all()


def test_norm_quant_per_tensor_zero_tensor():
    x = torch.zeros(5, 1024, dtype=torch.float16)
    xq, xs = sq.sq_norm_quant_per_tensor(_cuda(x), "none")
    torch.cuda.synchronize()
    assert not host(xq).any() and not host(xs).any()


@pytest.mark.parametrize("k", [64, 4096, 20480, 133120])
def test_static_step(k):
    g = torch.Generator().manual_seed(k)
    a = (torch.rand(k, generator=g) * 50).float()
    a[k // 3] = 900.0
    s = (torch.rand(k, generator=g) * 4 + 0.05).float()
    st = sq.sq_static_step(_cuda(a), _cuda(s))
    torch.cuda.synchronize()
    assert bits(O.static_step(a.numpy(), s.numpy()).reshape(1)) == bits(host(st))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("nk", [(48, 512), (300, 4096), (2100, 1024), (64, 81920)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_fold_per_tensor(dtype, norm, nk):
    n, k = nk
    seed = _seed("foldt", dtype, norm, n, k)
    g = torch.Generator().manual_seed(seed)
    a = (torch.rand(k, generator=g) * 5 + 0.01).float()
    a[:: max(1, k // 7)] *= 40.0
    w = (torch.randn(n, k, generator=g) * 0.02).to({"f32": torch.float32, "f16": torch.float16,
                                                     "bf16": torch.bfloat16}[dtype])
    gamma, beta = _params(k, seed + 1, norm)
    if norm == "none":
        gamma = beta = None
    out = sq.smoothquant_fold_per_tensor(_cuda(a), _cuda(w), 0.5, 1e-5, norm, _cuda(gamma), _cuda(beta))
    torch.cuda.synchronize()
    w_np = to_numpy(w)
    s_ref, dist, other = O.smoothing_factors(a.numpy(), O.weight_colmax(w_np, dtype), 0.5, 1e-5)
    s_gpu = host(out["s"])
    diff = bits(s_ref) != bits(s_gpu)
    if diff.any():                                      # either neighbour of a near-tie s is a correct rounding
        assert ((dist < O.smoothquant_oracle.NEAR_TIE) & (bits(other) == bits(s_gpu)))[diff].all()
        s_ref = np.where(diff, other, s_ref)
    f = O.fold_per_tensor(a.numpy(), w_np, dtype, 0.5, 1e-5, norm, _np(gamma), _np(beta), s=s_ref)
    assert np.array_equal(bits(f["gamma_f"]), bits(host(out["gamma_f"])))
    if f["beta_f"] is not None:
        assert np.array_equal(bits(f["beta_f"]), bits(host(out["beta_f"])))
    assert np.array_equal(bits(f["w_scale"]), bits(host(out["w_scale"])))
    assert np.array_equal(f["wq"], host(out["wq"]))


def test_static_pipeline_end_to_end():
    """Calibrate -> per-tensor fold -> static step -> static quantisation -> GEMM. Each stage is checked
    against the oracle fed with the HIP path's output of the stage before (near-ties in the norm
    statistics may legitimately round either way, so the stages are chained on the GPU's choices)."""
    m, k, n, mc = 64, 4096, 1024, 256
    x, gamma, beta = _inputs("e2e", "f16", "layernorm", m, k)
    xc, _, _ = _inputs("e2e-cal", "f16", "layernorm", mc, k)
    g = torch.Generator().manual_seed(17)
    w = (torch.randn(n, k, generator=g) * 0.02).half()
    amax = sq.smoothquant_calibrate(_cuda(xc), "layernorm", _cuda(gamma), _cuda(beta), 1e-5)
    fo = sq.smoothquant_fold_per_tensor(amax, _cuda(w), 0.5, 1e-5, "layernorm", _cuda(gamma), _cuda(beta))
    st = sq.sq_static_step(amax, fo["s"])
    xq, xs = sq.sq_norm_quant_static(_cuda(x), st, "layernorm", fo["gamma_f"], fo["beta_f"], 1e-5)
    y = sq.sq_w8a8_gemm(xq, xs, fo["wq"], fo["w_scale"], out_dtype=torch.float16)
    torch.cuda.synchronize()
    a_gpu = host(amax)
    check_calibrate(to_numpy(xc), "f16", "layernorm", gamma.numpy(), beta.numpy(), 1e-5, a_gpu, label="e2e")
    s_ref, dist, other = O.smoothing_factors(a_gpu, O.weight_colmax(to_numpy(w), "f16"), 0.5, 1e-5)
    s_gpu = host(fo["s"])
    diff = bits(s_ref) != bits(s_gpu)
    assert ((dist < O.smoothquant_oracle.NEAR_TIE) & (bits(other) == bits(s_gpu)))[diff].all()
    f = O.fold_per_tensor(a_gpu, to_numpy(w), "f16", 0.5, 1e-5, "layernorm", gamma.numpy(), beta.numpy(), s=s_gpu)
    assert np.array_equal(f["wq"], host(fo["wq"])) and np.array_equal(bits(f["w_scale"]), bits(host(fo["w_scale"])))
    step = O.static_step(a_gpu, s_gpu)
    assert bits(np.array([step], F32)) == bits(host(st))
    q, xsr, info = O.norm_quant_per_tensor(to_numpy(x), "f16", "layernorm", f["gamma_f"], f["beta_f"], 1e-5,
                                           step=step)
    _compare(q, xsr, info, host(xq), host(xs), "e2e",
             (to_numpy(x), "f16", "layernorm", f["gamma_f"], f["beta_f"], 1e-5))
    y_ref, _ = O.dequantize(O.int_gemm(host(xq), f["wq"]), xsr, f["w_scale"], None, "f16")
    assert np.array_equal(bits(y_ref), bits(host(y)))
