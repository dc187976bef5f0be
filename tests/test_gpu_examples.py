"""The pages' worked examples through the HIP kernels (needs an MI355X): the printed steps, codes and
level counts, from the golden fixtures the oracle's pins use, and the codes against the oracle's."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import w8a8_int8_linear_amd as sq
from tests.gpu_check import bits, host

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_page3_outlier_row():
    """One 4096-wide token with two outlier channels: step 60/127, 45 -> 95, -60 -> -127, the
    ordinary channels on 9 levels, and a 30x finer step once the outliers are gone."""
    g = _golden("p3_fix1_outlier_row.json")
    k, pr, tol = g["row"]["k"], g["printed"], g["printed_precision"]
    rng = np.random.default_rng(5)
    row = rng.uniform(g["row"]["ordinary_low"], g["row"]["ordinary_high"], k).astype(F32)
    row[0], row[1] = g["row"]["ordinary_high"], g["row"]["ordinary_low"]
    for ch, v in g["row"]["outliers"].items():
        row[int(ch)] = v
    xq, xs = sq.sq_norm_quant(_cuda(row[None, :]), "none")
    torch.cuda.synchronize()
    q, step = host(xq)[0], host(xs)[0]
    assert step == F32(60.0) / F32(127.0)
    assert abs(float(step) - pr["step_with_outliers"]) < tol["step_with_outliers"]
    assert q[1512] == 95 and q[2817] == -127
    ordinary = np.delete(q, [1512, 2817])
    assert len(np.unique(ordinary)) == pr["ordinary_levels"] and ordinary.min() == -4 and ordinary.max() == 4
    q_ref, s_ref, _ = O.norm_quant(row[None, :], "f32", O.NONE)
    assert np.array_equal(q_ref[0], q) and bits(s_ref)[0] == bits(np.array([step], F32))[0]
    # without the outliers (two zero channels keep K a multiple of 64 and leave the row max alone)
    row2 = np.concatenate([np.delete(row, [1512, 2817]), np.zeros(2, F32)])
    _, xs2 = sq.sq_norm_quant(_cuda(row2[None, :]), "none")
    torch.cuda.synchronize()
    step2 = float(host(xs2)[0])
    assert abs(step2 - pr["step_without_outliers"]) < tol["step_without_outliers"]
    assert float(step) / step2 == pytest.approx(pr["finer_factor"], rel=1e-6)


def test_page4_two_channel_example():
    """Two channels with activation maxima 60 and 1, weight maxima 0.2 and 0.5 (padded with zero
    channels to K = 64, which changes no per-channel result): about 2 levels for channel 2 before
    smoothing, about 26 at alpha 0.5 (step 3.46/127) and about 67 at alpha 0.8, with a 12.7x weight range."""
    g = _golden("p4_two_channel_example.json")
    pr, tol = g["printed"], g["printed_precision"]
    act, wmax = g["act_max"], g["w_max"]
    k = 64
    x_cal = np.zeros((2, k), F32)
    x_cal[0, :2], x_cal[1, :2] = [act[0], -0.5], [-3.0, act[1]]
    w = np.zeros((3, k), F32)
    w[:, :2] = [[wmax[0], -0.1], [0.05, wmax[1]], [-0.2, 0.25]]
    a = sq.smoothquant_calibrate(_cuda(x_cal), "none")
    torch.cuda.synchronize()
    a_h = host(a)
    assert a_h[:2].tolist() == [60.0, 1.0] and not a_h[2:].any()
    step0 = float(a_h.max()) / 127
    assert abs(step0 - pr["before"]["step"]) < tol["step"]
    assert abs(float(a_h[1]) / step0 - pr["before"]["channel2_levels"]) < tol["levels"] + 0.2
    for key, alpha in [("alpha_0.5", 0.5), ("alpha_0.8", 0.8)]:
        fo = sq.smoothquant_fold(a, _cuda(w), alpha)
        # the smoothed calibration maxima a_j / s_j as one token through the quantiser (gamma' = 1/s)
        xq, xs = sq.sq_norm_quant(a[None, :].contiguous(), "none", fo["gamma_f"])
        torch.cuda.synchronize()
        q, step, s = host(xq)[0], float(host(xs)[0]), host(fo["s"])
        assert int(q[1]) == pr[key]["channel2_levels"]                   # "about 26" / "about 67" levels
        if "step" in pr[key]:
            assert abs(step * 127 - pr[key]["step_numerator"]) < tol["step_numerator"]
            assert abs(step - pr[key]["step"]) < tol["step"]
        if "weight_range" in pr[key]:
            rng_w = (wmax[0] * float(s[0])) / (wmax[1] * float(s[1]))
            assert abs(rng_w - pr[key]["weight_range"]) < tol["weight_range"]
        f = O.fold(a_h, w, "f32", alpha)
        assert np.array_equal(bits(f["s"]), bits(s)) and np.array_equal(f["wq"], host(fo["wq"]))
