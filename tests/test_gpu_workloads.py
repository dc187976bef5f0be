"""The whole layer on the five workloads (calibrate -> fold -> norm+quantise -> GEMM),
all on the GPU, checked stage by stage against the oracle run on the same inputs.

Small workloads are checked in full; at full size the check samples token rows
and weight rows (every stage is row-independent) and checks every channel of
the smoothing factors and folded norm parameters.
"""
import numpy as np
import pytest
import torch

import oracle as O
import w8a8_int8_linear_amd as sq
from synth import WORKLOADS, site_inputs, to_numpy
from tests.gpu_check import check_calibrate, check_fold, check_norm_quant, check_output, host

pytestmark = pytest.mark.gpu
OUT_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
EPS = 1e-5


def _rows(n, cap, seed):
    if n <= cap:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    pick = rng.choice(n - 2, cap - 2, replace=False) + 1
    return np.sort(np.concatenate([[0, n - 1], pick]))          # first and last rows included


def _gather(t, rows):
    return t[torch.as_tensor(rows, device=t.device)]


def run_site(wl_id, site_idx, m, x_rows_cap=256, w_rows_cap=512):
    wl = WORKLOADS[wl_id]
    site = wl.sites[site_idx]
    norm = site.norm
    inp = site_inputs(wl_id, site_idx, m=m, device="cuda")
    print(f"\n[{wl.name} {site.name} M={m} N={site.n} K={site.k}] GPU chain", flush=True)
    a = sq.smoothquant_calibrate(inp["x_cal"], norm, inp["gamma"], inp["beta"], EPS)
    f = sq.smoothquant_fold(a, inp["w"], wl.alpha, 1e-5, norm, inp["gamma"], inp["beta"])
    xq, xs = sq.sq_norm_quant(inp["x"], norm, f["gamma_f"], f["beta_f"], EPS)
    y = sq.sq_w8a8_gemm(xq, xs, f["wq"], f["w_scale"], out_dtype=OUT_DT[wl.out_dtype])
    torch.cuda.synchronize()

    gamma = None if inp["gamma"] is None else host(inp["gamma"])
    beta = None if inp["beta"] is None else host(inp["beta"])
    a_ref = check_calibrate(to_numpy(inp["x_cal"]), wl.dtype, norm, gamma, beta, EPS, host(a), label="calibrate")
    w_rows = _rows(site.n, w_rows_cap, 1)
    fold_gpu = dict(f, wq=_gather(f["wq"], w_rows), w_scale=_gather(f["w_scale"], w_rows))
    w_np = to_numpy(inp["w"])
    fref, s_ties = check_fold(a_ref, w_np, wl.dtype, wl.alpha, 1e-5, norm, gamma, beta, fold_gpu, rows=w_rows,
                              label="fold")
    del w_np
    x_rows = _rows(m, x_rows_cap, 2)
    x_np = to_numpy(_gather(inp["x"], x_rows))
    ties = check_norm_quant(x_np, wl.dtype, norm, fref["gamma_f"], fref["beta_f"], EPS,
                            host(_gather(xq, x_rows)), host(_gather(xs, x_rows)), label="norm_quant")
    # outputs at every sampled (token, channel) pair, from the codes and steps check_norm_quant has just
    # accepted: the oracle's own, or on a near-tie row one of the row's correct roundings
    acc = O.int_gemm(host(_gather(xq, x_rows)), fref["wq"])
    out_ref, v32 = O.dequantize(acc, host(_gather(xs, x_rows)), fref["w_scale"], None, wl.out_dtype)
    y_sel = _gather(_gather(y, x_rows).t().contiguous(), w_rows).t().contiguous()
    check_output(host(y_sel), out_ref, v32, wl.out_dtype, label="gemm")
    print(f"  ok: {len(x_rows)} token rows, {len(w_rows)} weight rows checked; near-ties s={s_ties} rows={ties}",
          flush=True)


@pytest.mark.parametrize("wl_id,site_idx,m", [
    (1, 0, 16), (2, 0, 2048), (2, 1, 2048), (3, 0, 1), (3, 0, 8), (3, 0, 32), (3, 0, 64), (3, 1, 1), (3, 1, 8),
    (3, 1, 32), (3, 1, 64), (4, 0, 4096), (4, 1, 4096)])
def test_workload_site(wl_id, site_idx, m):
    run_site(wl_id, site_idx, m)


@pytest.mark.parametrize("site_idx", [0, 1])
def test_workload5_full_size(site_idx):
    run_site(5, site_idx, 8192, x_rows_cap=24, w_rows_cap=128)
