"""The synthetic accuracy study (plain INT8 and FP8 against SmoothQuant over alpha): its binary64
reference and its level metrics on the CPU, and on the GPU the construction it uses for plain
INT8 (s = 1 exactly) and the agreement of its hot-path errors with the oracle's pipeline."""
import numpy as np
import pytest
import torch

import bench
import oracle as O
from tests.gpu_check import check_norm_quant


@pytest.mark.parametrize("norm", ["none", "layernorm", "rmsnorm"])
def test_reference_linear_matches_numpy_binary64(norm):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)).astype(np.float32) * 3
    w = rng.standard_normal((7, 64)).astype(np.float32) * 0.02
    g = (1 + 0.1 * rng.standard_normal(64)).astype(np.float32)
    b = (0.1 * rng.standard_normal(64)).astype(np.float32)
    got = bench.reference_linear(torch, torch.from_numpy(x), norm, torch.from_numpy(g), torch.from_numpy(b),
                                 torch.from_numpy(w)).numpy()
    x64 = x.astype(np.float64)
    if norm == "layernorm":
        y = (x64 - x64.mean(1, keepdims=True)) / np.sqrt(x64.var(1, keepdims=True) + 1e-5) * g + b
    elif norm == "rmsnorm":
        y = x64 / np.sqrt((x64 ** 2).mean(1, keepdims=True) + 1e-5) * g
    else:
        y = x64
    assert np.allclose(got, y @ w.astype(np.float64).T, rtol=1e-12, atol=1e-15)


def test_ordinary_span():
    xq = torch.tensor([[3, -120, 5, 0], [1, 127, -7, 2], [0, 90, 2, -1]], dtype=torch.int8)
    # channel 1 is the outlier; the rest reach 5, 7, 2 -> median 5
    assert bench.ordinary_span(xq, [1]) == 5


def test_ordinary_span_fp8():
    # E4M3 codes: 0x38 = 1, 0x40 = 2, 0x48 = 4, 0x30 = 0.5, 0x01 = 2^-9, 0xB8 = -1, 0x7E = 448
    xq = torch.tensor([[0x38, 0x7E, 0x40, 0x00], [0xB8, 0x7E, 0x30, 0x01], [0x00, 0xFE, 0x48, 0x00]], dtype=torch.uint8)
    # channel 1 is the outlier; the rest reach 2, 1, 4 -> median 2
    assert bench.ordinary_span_fp8(xq, [1]) == 2.0


@pytest.mark.gpu
def test_study_plain_fold_gives_unit_s_and_matches_oracle():
    import w8a8_int8_linear_amd as sq
    from synth import WORKLOADS, site_inputs, to_numpy
    wl = WORKLOADS[2]
    inp = site_inputs(wl.id, 0, m=64, device="cuda")
    w, x, g, b = inp["w"], inp["x"], inp["gamma"], inp["beta"]
    wmax = sq.smoothquant_calibrate(w, "none")
    fo = sq.smoothquant_fold(wmax, w, 0.5, 1e-5, "layernorm", g, b)
    assert (fo["s"] == 1.0).all()                                   # plain INT8: no smoothing at all
    assert torch.equal(fo["gamma_f"], g) and torch.equal(fo["beta_f"], b)
    recs = bench.accuracy_site(torch, sq, wl, 0, 64)
    get = {(r["scheme"], r["alpha"]): r for r in recs}
    plain = get[("plain INT8, per-tensor X and W", None)]["rel_err"]
    assert get[("SmoothQuant O2: per-tensor X and W", 0.5)]["rel_err"] < plain / 2
    assert get[("SmoothQuant, per-token X, per-channel W", 0.5)]["rel_err"] < plain / 2
    # the hot-path scheme at alpha 0.5 through the oracle gives the same error (its outputs are bit-identical)
    amax = sq.smoothquant_calibrate(inp["x_cal"], "layernorm", g, b, 1e-5)
    f = O.fold(amax.cpu().numpy(), to_numpy(w), wl.dtype, 0.5, 1e-5, "layernorm", g.cpu().numpy(), b.cpu().numpy(),
               s=sq.smoothquant_fold(amax, w, 0.5, 1e-5, "layernorm", g, b)["s"].cpu().numpy())
    # the GPU's codes, checked against the oracle (either rounding of a near-tie row is correct)
    xq_g, xs_g = sq.sq_norm_quant(x, "layernorm", torch.from_numpy(f["gamma_f"]).cuda(),
                                  torch.from_numpy(f["beta_f"]).cuda(), 1e-5)
    q, xs = xq_g.cpu().numpy(), xs_g.cpu().numpy()
    check_norm_quant(to_numpy(x), wl.dtype, "layernorm", f["gamma_f"], f["beta_f"], 1e-5, q, xs, label="study")
    y, _ = O.dequantize(O.int_gemm(q, f["wq"]), xs, f["w_scale"], None, "f32")
    y_ref = bench.reference_linear(torch, x.cpu(), "layernorm", g.cpu(), b.cpu(), w.cpu())
    err = torch.linalg.norm(torch.from_numpy(y).double() - y_ref).item() / torch.linalg.norm(y_ref).item()
    # (the binary64 references differ only in summation order; the study rounds to 4 digits)
    assert err == pytest.approx(get[("SmoothQuant, per-token X, per-channel W", 0.5)]["rel_err"], rel=1e-3)
