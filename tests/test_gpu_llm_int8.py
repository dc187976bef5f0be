"""The LLM.int8() decomposition on the HIP path against oracle.llm_int8 (needs an MI355X).

Small cases are checked in full: the call's per-channel maxima, the outlier set, the masked norm
parameters, the INT8 codes and steps, the 16-bit operands and deq bit for bit, and the output within
the bound of a binary32 evaluation of deq + the 16-bit product. Full-size workload sites are checked on
sampled token and weight rows against the outlier set the whole batch gave, that set itself against
a binary64 evaluation of every row."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import oracle.llm_int8 as L
import w8a8_int8_linear_amd as sq
from synth import WORKLOADS, rand_tokens, site_inputs, to_numpy
from tests.gpu_check import bits, check_calibrate, check_llm_int8, host

pytestmark = pytest.mark.gpu
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
EPS = 1e-5


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def _params(k, seed, norm):
    if norm == "none":
        return None, None
    g = torch.Generator().manual_seed(seed)
    gamma = (1 + 0.1 * torch.randn(k, generator=g)).float()
    beta = (0.1 * torch.randn(k, generator=g)).float() if norm == "layernorm" else None
    return gamma, beta


def _weights_on_gpu(w, w_dtype, label):
    """Offline per-output-channel INT8 of w on the GPU (the norm-free quantiser), against the oracle."""
    wq, ws = sq.sq_norm_quant(w, "none")
    torch.cuda.synchronize()
    wq_ref, ws_ref = L.weights(to_numpy(w), w_dtype)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(bits(host(ws)), bits(ws_ref)), label
    return wq, ws


def _check_masks(parts, gamma, beta, k, label):
    o = np.zeros(k, bool)
    o[host(parts["idx"]).astype(np.int64)] = True
    g = np.ones(k, np.float32) if gamma is None else _np(gamma)
    assert np.array_equal(bits(host(parts["gamma_m"])), bits(np.where(o, np.float32(0), g))), label
    if beta is not None:
        assert np.array_equal(bits(host(parts["beta_m"])), bits(np.where(o, np.float32(0), _np(beta)))), label


def _run(x, w, norm, gamma, beta, tau, out, bias=None, label=""):
    w_dtype = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[w.dtype]
    wq, ws = _weights_on_gpu(w, w_dtype, label)
    y, work = sq.sq_llm_int8_linear(x, w, wq, ws, norm, gamma, beta, EPS, tau, bias, TORCH_DT[out])
    torch.cuda.synchronize()
    m, k = x.shape
    return y, sq.llm_int8_parts(work, m, w.shape[0], k, w.dtype), w_dtype


# (dtype, norm, M, K, N, outlier channels, outlier scale, out dtype, tau, bias)
CASES = [
    ("f16", "layernorm", 200, 4096, 520, 4, 30.0, "f16", 6.0, False),       # tiled INT8 GEMM, ragged M and N
    ("f16", "none", 37, 512, 300, 41, 30.0, "f32", 6.0, True),              # decode GEMM, |O| = 41 (P = 64), bias
    ("bf16", "rmsnorm", 130, 1024, 1030, 8, 40.0, "bf16", 6.0, False),      # bf16 operands, N % 4 != 0
    ("f32", "none", 16, 512, 512, 4, 50.0, "f32", 6.0, False),              # the tiny linear's shape
    ("f16", "none", 65, 320, 200, 3, 30.0, "f16", 6.0, False),              # K % 128 == 64
    ("f16", "layernorm", 64, 4096, 4096, 6, 40.0, "f16", math.inf, False),  # no outlier: per-token W8A8
    ("f16", "rmsnorm", 33, 256, 100, 0, 1.0, "f32", 0.0, False),            # every channel an outlier
    ("bf16", "layernorm", 1, 9216, 9216, 6, 40.0, "bf16", 6.0, False),      # one token, OPT-66B width
    ("f16", "layernorm", 300, 2048, 2000, 70, 30.0, "f16", 6.0, True),      # |O| = 70 (P = 96), bias
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}x{c[4]}-o{c[5]}-t{c[8]}")
def test_llm_int8_parity(case):
    dtype, norm, m, k, n, n_out, scale, out, tau, with_bias = case
    label = f"{dtype}/{norm}/{m}x{k}x{n}"
    seed = zlib_seed(label)
    x = rand_tokens(m, k, dtype, seed, n_outliers=n_out, outlier_scale=scale)
    gamma, beta = _params(k, seed + 1, norm)
    w = (rand_tokens(n, k, "f32", seed + 2) * 0.02).to(TORCH_DT[dtype])
    bias = rand_tokens(1, n, "f32", seed + 3)[0] if with_bias else None
    cu = (lambda t: None if t is None else t.cuda())
    print(f"\n[{label} tau={tau}] GPU", flush=True)
    y, parts, w_dtype = _run(cu(x), cu(w), norm, cu(gamma), cu(beta), tau, out, cu(bias), label)
    x_np, w_np = to_numpy(x), to_numpy(w)
    g_np, b_np = _np(gamma), _np(beta)
    check_calibrate(x_np, dtype, norm, g_np, b_np, EPS, host(parts["absmax"]), label=label)
    assert np.array_equal(host(parts["idx"]).astype(np.int64),
                          np.where(host(parts["absmax"]) >= np.float32(tau))[0]), f"{label}: O != {{absmax >= tau}}"
    _check_masks(parts, gamma, beta, k, label)
    if norm != "none":
        st = host(parts["stats"])
        for r in range(m):
            s = O.row_stats(O.widen(x_np[r], dtype), norm)
            r32 = np.float32(1) / np.sqrt(np.float32(s["var"]) + np.float32(EPS))
            assert st[r, 1] == r32 or s["var_dist"] < O.smoothquant_oracle.NEAR_TIE, f"{label}: rstd row {r}"
    _, worst = check_llm_int8(x_np, dtype, norm, g_np, b_np, EPS, tau, w_np, w_dtype, out, parts, host(y),
                              bias=_np(bias), label=label)
    if tau == math.inf:
        assert parts["count"] == 0
    if tau == 0.0:
        assert parts["count"] == k and not host(parts["xq"]).any()
    print(f"  ok: |O| = {parts['count']}, worst error {worst:.3g} of the bound", flush=True)


def zlib_seed(label):
    import zlib
    return zlib.crc32(label.encode()) & 0xFFFFF


def test_page3_token_through_the_gpu():
    """The page's token (4,096 values in [-2, 2], channels 1512 = 45 and 2817 = -60) goes through the
    decomposition: those two channels take the 16-bit lane, the rest a step of 2/127."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "p3_fix1_outlier_row.json")) as f:
        g = json.load(f)
    k = g["row"]["k"]
    rng = np.random.default_rng(5)
    row = rng.uniform(g["row"]["ordinary_low"], g["row"]["ordinary_high"], k).astype(np.float32)
    row[0], row[1] = g["row"]["ordinary_high"], g["row"]["ordinary_low"]
    for ch, v in g["row"]["outliers"].items():
        row[int(ch)] = v
    x = torch.from_numpy(np.repeat(row[None, :], 4, axis=0)).cuda()
    w = (torch.randn(64, k, generator=torch.Generator().manual_seed(7)) * 0.02).half().cuda()
    y, parts, _ = _run(x, w, "none", None, None, 6.0, "f32", label="p3")
    assert host(parts["idx"]).tolist() == [1512, 2817]
    assert (host(parts["x_scale"]) == np.float32(2.0) / np.float32(127.0)).all()
    assert host(parts["x16"])[:, :2].astype(np.float32).tolist() == [[45.0, -60.0]] * 4
    check_llm_int8(np.repeat(row[None, :], 4, axis=0), "f32", "none", None, None, EPS, 6.0, to_numpy(w), "f16", "f32",
                   parts, host(y), label="p3")


def test_workspace_reuse_and_smaller_call():
    """The same workspace serves a second, smaller call: every part it reads is rewritten first."""
    x1 = rand_tokens(150, 1024, "f16", 91, n_outliers=9, outlier_scale=40.0).cuda()
    w = (rand_tokens(700, 1024, "f32", 92) * 0.02).half().cuda()
    wq, ws = sq.sq_norm_quant(w, "none")
    need = sq.sq_llm_int8_workspace(150, 700, 1024)["total"]
    work = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")        # garbage: nothing is read unwritten
    y1, _ = sq.sq_llm_int8_linear(x1, w, wq, ws, "none", tau=6.0, out_dtype=torch.float16, workspace=work)
    torch.cuda.synchronize()
    x2 = rand_tokens(20, 1024, "f16", 93, n_outliers=2, outlier_scale=40.0).cuda()
    y2, _ = sq.sq_llm_int8_linear(x2, w, wq, ws, "none", tau=6.0, out_dtype=torch.float16, workspace=work)
    torch.cuda.synchronize()
    parts = sq.llm_int8_parts(work, 20, 700, 1024, torch.float16)
    check_llm_int8(to_numpy(x2), "f16", "none", None, None, EPS, 6.0, to_numpy(w), "f16", "f16", parts, host(y2),
                   label="second call")
    y1b, _ = sq.sq_llm_int8_linear(x1, w, wq, ws, "none", tau=6.0, out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y1b)                                   # the same call in a fresh workspace


# --------------------------------------------------------------------------- full-size workload sites

def _approx_outliers(x, norm, gamma, beta, tau, chunk=512):
    """max_t |y_tj| in binary64 over every row (chunked on the host), y the norm with the model's
    gamma, beta: within about 1e-6 relative of the binary32 y the kernels compute."""
    m, k = x.shape
    amax = np.zeros(k)
    g = np.ones(k) if gamma is None else gamma.astype(np.float64)
    b = np.zeros(k) if beta is None else beta.astype(np.float64)
    for r0 in range(0, m, chunk):
        xs = x[r0:r0 + chunk].float().cpu().numpy().astype(np.float64)
        if norm == "layernorm":
            mu = xs.mean(axis=1, keepdims=True)
            y = (xs - mu) / np.sqrt(((xs - mu) ** 2).mean(axis=1, keepdims=True) + EPS) * g + b
        elif norm == "rmsnorm":
            y = xs / np.sqrt((xs * xs).mean(axis=1, keepdims=True) + EPS) * g
        else:
            y = xs
        amax = np.maximum(amax, np.abs(y).max(axis=0))
    return amax


def _sample(n, cap, seed):
    if n <= cap:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([[0, n - 1], rng.choice(n - 2, cap - 2, replace=False) + 1]))


@pytest.mark.parametrize("wl_id,site_idx,m", [(2, 0, 2048), (2, 1, 2048), (3, 0, 1), (3, 1, 64), (4, 0, 4096),
                                              (5, 0, 8192), (5, 1, 8192)])
def test_llm_int8_workload_site(wl_id, site_idx, m):
    wl = WORKLOADS[wl_id]
    site = wl.sites[site_idx]
    inp = site_inputs(wl_id, site_idx, m=m, device="cuda")
    label = f"{wl.name} {site.name} M={m}"
    print(f"\n[{label}] GPU", flush=True)
    y, parts, w_dtype = _run(inp["x"], inp["w"], site.norm, inp["gamma"], inp["beta"], L.TAU, wl.out_dtype,
                             label=label)
    gamma, beta = _np(inp["gamma"]), _np(inp["beta"])
    # the outlier set, against a binary64 evaluation of every row (channels near tau are left open)
    a64 = _approx_outliers(inp["x"], site.norm, gamma, beta, L.TAU)
    a_gpu = host(parts["absmax"]).astype(np.float64)
    # relative near tau and above; absolute below 1, where a single token's y can cancel to ~0
    assert np.all(np.abs(a_gpu - a64) <= 1e-5 * np.maximum(a64, 1.0)), f"{label}: absmax"
    o_gpu = host(parts["idx"]).astype(np.int64)
    assert np.array_equal(o_gpu, np.where(a_gpu >= L.TAU)[0])
    sure = np.abs(a64 - L.TAU) > 1e-4 * L.TAU
    member = np.zeros(site.k, bool)
    member[o_gpu] = True
    assert np.array_equal(member[sure], (a64 >= L.TAU)[sure]), f"{label}: outlier set"
    if m >= 64:            # with a few tokens a planted channel's own draws may all stay below tau
        assert set(inp["outliers"].tolist()) <= set(o_gpu.tolist()), f"{label}: a planted outlier channel is missing"
    _check_masks(parts, inp["gamma"], inp["beta"], site.k, label)
    # sampled token rows x sampled weight rows, bit for bit against the oracle with the batch's set
    rows = _sample(m, 24, 1)
    w_rows = _sample(site.n, 128, 2)
    sub = dict(parts)
    for key in ("xq", "x_scale", "x16", "stats"):
        sub[key] = parts[key][torch.as_tensor(rows, device="cuda")]
    sub["w16"] = parts["w16"][torch.as_tensor(w_rows, device="cuda")]
    sub["deq"] = parts["deq"][torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(w_rows, device="cuda")]
    y_sel = y[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(w_rows, device="cuda")]
    x_np = to_numpy(inp["x"][torch.as_tensor(rows, device="cuda")])
    w_np = to_numpy(inp["w"][torch.as_tensor(w_rows, device="cuda")])
    _, worst = check_llm_int8(x_np, wl.dtype, site.norm, gamma, beta, EPS, L.TAU, w_np, w_dtype, wl.out_dtype, sub,
                              host(y_sel), outliers=o_gpu, label=label)
    print(f"  ok: |O| = {parts['count']} (planted {len(inp['outliers'])}), {len(rows)} x {len(w_rows)} outputs, "
          f"worst error {worst:.3g} of the bound", flush=True)
