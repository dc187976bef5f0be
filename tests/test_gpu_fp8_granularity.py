"""Per-tensor FP8 (OCP E4M3) steps on the HIP path against the oracle (needs an MI355X): one dynamic
step for the whole activation tensor, a static calibrated step with saturation at +-448, the static
step itself, and the fold with one weight step. Codes, steps and scale vectors bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import w8a8_int8_linear_amd as sq
from synth import to_numpy
from tests.gpu_check import bits, check_calibrate, host
from tests.test_gpu_fp8 import fp8_gemm_tolerance
from tests.test_gpu_granularity import SHAPES, _compare, _cuda, _inputs, _np, _params, _seed

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_norm_quant_fp8_per_tensor(dtype, norm, shape):
    m, k = shape
    x, gamma, beta = _inputs("nq8t", dtype, norm, m, k)
    xq, xs = sq.sq_norm_quant_fp8_per_tensor(_cuda(x), norm, _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    q, xsr, info = O.norm_quant_fp8_per_tensor(to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5)
    _compare(q, xsr, info, host(xq), host(xs), f"{dtype}/{norm}/{m}x{k}",
             (to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5), fp8=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("shape", [(7, 512), (33, 4096), (3, 20480), (2, 81920)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("factor", [0.37, 1.0, 2.5])
def test_norm_quant_fp8_static(dtype, norm, shape, factor):
    # factor < 1: a step below the tensor's own, so the largest values saturate at 448
    m, k = shape
    x, gamma, beta = _inputs("nq8s", dtype, norm, m, k)
    _, xs_dyn, _ = O.norm_quant_fp8_per_tensor(to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5)
    step = F32(xs_dyn[0] * F32(factor))
    st = torch.tensor([step], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_fp8_static(_cuda(x), st, norm, _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    q, xsr, info = O.norm_quant_fp8_per_tensor(to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5, step=step)
    _compare(q, xsr, info, host(xq), host(xs), f"{dtype}/{norm}/{m}x{k}/x{factor}",
             (to_numpy(x), dtype, norm, _np(gamma), _np(beta), 1e-5), fp8=True)
    codes = host(xq)
    assert not np.isin(codes, [0x7F, 0xFF]).any()                       # saturation, never NaN
    if factor < 1:
        assert np.isin(codes, [0x7E, 0xFE]).sum() > 1                      # saturation happened


def test_norm_quant_fp8_static_saturates_far_beyond_range():
    # values up to 10^4 times the step's range: every one of them takes the largest code
    x = np.zeros((3, 512), F32)
    x[0, :4] = [1e5, -1e5, 448.0, 449.0]
    x[1, ::2] = 3e6
    x[2] = np.linspace(-2000, 2000, 512).astype(F32)
    st = torch.tensor([1.0], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_fp8_static(_cuda(torch.from_numpy(x)), st, "none")
    torch.cuda.synchronize()
    q, xsr, _ = O.norm_quant_fp8_per_tensor(x, "f32", "none", step=F32(1.0))
    assert np.array_equal(q, host(xq)) and np.array_equal(bits(xsr), bits(host(xs)))
    assert host(xq)[0, :4].tolist() == [0x7E, 0xFE, 0x7E, 0x7E]


@pytest.mark.parametrize("step", [0.0, -1.0])
def test_norm_quant_fp8_static_nonpositive_step_gives_zero_codes(step):
    x, gamma, beta = _inputs("nq8z", "f16", "layernorm", 9, 4096)
    st = torch.tensor([step], dtype=torch.float32, device="cuda")
    xq, xs = sq.sq_norm_quant_fp8_static(_cuda(x), st, "layernorm", _cuda(gamma), _cuda(beta), 1e-5)
    torch.cuda.synchronize()
    assert not host(xq).any()
    assert (host(xs) == F32(step)).all()


@pytest.mark.parametrize("k", [64, 4096, 20480, 133120])
def test_static_step_fp8(k):
    g = torch.Generator().manual_seed(k + 1)
    a = (torch.rand(k, generator=g) * 50).float()
    a[k // 3] = 900.0
    s = (torch.rand(k, generator=g) * 4 + 0.05).float()
    st = sq.sq_static_step_fp8(_cuda(a), _cuda(s))
    torch.cuda.synchronize()
    assert bits(O.static_step_fp8(a.numpy(), s.numpy()).reshape(1)) == bits(host(st))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
@pytest.mark.parametrize("nk", [(48, 512), (300, 4096), (2100, 1024), (64, 81920)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_fold_fp8_per_tensor(dtype, norm, nk):
    n, k = nk
    seed = _seed("fold8t", dtype, norm, n, k)
    g = torch.Generator().manual_seed(seed)
    a = (torch.rand(k, generator=g) * 5 + 0.01).float()
    a[:: max(1, k // 7)] *= 40.0
    w = (torch.randn(n, k, generator=g) * 0.02).to({"f32": torch.float32, "f16": torch.float16,
                                                     "bf16": torch.bfloat16}[dtype])
    gamma, beta = _params(k, seed + 1, norm)
    if norm == "none":
        gamma = beta = None
    out = sq.smoothquant_fold_fp8_per_tensor(_cuda(a), _cuda(w), 0.5, 1e-5, norm, _cuda(gamma), _cuda(beta))
    torch.cuda.synchronize()
    w_np = to_numpy(w)
    s_ref, dist, other = O.smoothing_factors(a.numpy(), O.weight_colmax(w_np, dtype), 0.5, 1e-5)
    s_gpu = host(out["s"])
    diff = bits(s_ref) != bits(s_gpu)
    if diff.any():                                      # either neighbour of a near-tie s is a correct rounding
        assert ((dist < O.smoothquant_oracle.NEAR_TIE) & (bits(other) == bits(s_gpu)))[diff].all()
        s_ref = np.where(diff, other, s_ref)
    f = O.fold_fp8_per_tensor(a.numpy(), w_np, dtype, 0.5, 1e-5, norm, _np(gamma), _np(beta), s=s_ref)
    assert np.array_equal(bits(f["gamma_f"]), bits(host(out["gamma_f"])))
    if f["beta_f"] is not None:
        assert np.array_equal(bits(f["beta_f"]), bits(host(out["beta_f"])))
    assert np.array_equal(bits(f["w_scale"]), bits(host(out["w_scale"])))
    assert np.array_equal(f["wq"], host(out["wq"]))


def test_fp8_static_pipeline_end_to_end():
    """Calibrate -> per-tensor FP8 fold -> static FP8 step -> static FP8 quantisation -> FP8 GEMM, each
    stage against the oracle fed with the HIP path's output of the stage before."""
    m, k, n, mc = 96, 4096, 1024, 256
    x, gamma, beta = _inputs("e2e8", "f16", "layernorm", m, k)
    xc, _, _ = _inputs("e2e8-cal", "f16", "layernorm", mc, k)
    g = torch.Generator().manual_seed(19)
    w = (torch.randn(n, k, generator=g) * 0.02).half()
    amax = sq.smoothquant_calibrate(_cuda(xc), "layernorm", _cuda(gamma), _cuda(beta), 1e-5)
    fo = sq.smoothquant_fold_fp8_per_tensor(amax, _cuda(w), 0.5, 1e-5, "layernorm", _cuda(gamma), _cuda(beta))
    st = sq.sq_static_step_fp8(amax, fo["s"])
    xq, xs = sq.sq_norm_quant_fp8_static(_cuda(x), st, "layernorm", fo["gamma_f"], fo["beta_f"], 1e-5)
    y = sq.sq_fp8_gemm(xq, xs, fo["wq"], fo["w_scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    a_gpu = host(amax)
    check_calibrate(to_numpy(xc), "f16", "layernorm", gamma.numpy(), beta.numpy(), 1e-5, a_gpu, label="e2e8")
    s_ref, dist, other = O.smoothing_factors(a_gpu, O.weight_colmax(to_numpy(w), "f16"), 0.5, 1e-5)
    s_gpu = host(fo["s"])
    diff = bits(s_ref) != bits(s_gpu)
    assert ((dist < O.smoothquant_oracle.NEAR_TIE) & (bits(other) == bits(s_gpu)))[diff].all()
    f = O.fold_fp8_per_tensor(a_gpu, to_numpy(w), "f16", 0.5, 1e-5, "layernorm", gamma.numpy(), beta.numpy(),
                              s=s_gpu)
    assert np.array_equal(f["wq"], host(fo["wq"])) and np.array_equal(bits(f["w_scale"]), bits(host(fo["w_scale"])))
    step = O.static_step_fp8(a_gpu, s_gpu)
    assert bits(np.array([step], F32)) == bits(host(st))
    q, xsr, info = O.norm_quant_fp8_per_tensor(to_numpy(x), "f16", "layernorm", f["gamma_f"], f["beta_f"], 1e-5,
                                               step=step)
    _compare(q, xsr, info, host(xq), host(xs), "e2e8",
             (to_numpy(x), "f16", "layernorm", f["gamma_f"], f["beta_f"], 1e-5), fp8=True)
    mi, ni = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    mi, ni = mi.ravel(), ni.ravel()
    acc, tol_acc = fp8_gemm_tolerance(host(xq), f["wq"], mi, ni)
    scale = host(xs).astype(np.float64)[mi] * f["w_scale"].astype(np.float64)[ni]
    err = np.abs(host(y)[mi, ni].astype(np.float64) - acc * scale)
    assert np.all(err <= tol_acc * scale * (1 + 2.0 ** -20) + (np.abs(acc) + tol_acc) * scale * 3 * 2.0 ** -24 + 1e-30)
