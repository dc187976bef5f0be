"""The hot path captured in a HIP graph (needs an MI355X).

Every entry point launches stream-ordered kernels only: the library allocates, copies, fills and
synchronises nothing. So a caller can capture a layer's quantiser + GEMM once and replay it, as a
serving loop does for its decode steps. Each case captures its chain with preallocated outputs. It
then replays the graph three times over fresh inputs copied into the captured input buffer, with eager
calls of the same entry points in between. Every replay must equal the eager result bit for bit (same
kernels, same inputs: the results are deterministic).
"""
import pytest
import torch

import w8a8_int8_linear_amd as sq
from synth import rand_tokens

pytestmark = pytest.mark.gpu
DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _bits(t):
    return t.view({1: torch.int8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def _norm_params(k, norm, seed):
    g = torch.Generator().manual_seed(seed)
    gamma = (1 + 0.1 * torch.randn(k, generator=g)).float().cuda() if norm != "none" else None
    beta = (0.1 * torch.randn(k, generator=g)).float().cuda() if norm == "layernorm" else None
    return gamma, beta


def _check_graph(chain, make_outs, inputs):
    """chain(x, outs) fills the tensors of outs; inputs are same-shaped tensors on the GPU."""
    eager = []
    for x in inputs:
        outs = make_outs()
        chain(x, outs)
        eager.append(outs)
    torch.cuda.synchronize()
    for i in range(1, len(inputs)):                  # a replay that kept its first input would be caught
        assert not torch.equal(_bits(eager[i][-1]), _bits(eager[0][-1]))
    static_x = inputs[0].clone()
    static_outs = make_outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                    # warm-up outside the capture
        chain(static_x, static_outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(static_x, static_outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, x in enumerate(inputs):
            static_x.copy_(x)
            torch.cuda.synchronize()
            graph.replay()
            scratch = make_outs()                    # eager work between the replays
            chain(inputs[(i + 1) % len(inputs)], scratch)
            torch.cuda.synchronize()
            for j, (got, want) in enumerate(zip(static_outs, eager[i])):
                assert torch.equal(_bits(got), _bits(want)), f"replay {rep}, input {i}, output {j}"
            for j, (got, want) in enumerate(zip(scratch, eager[(i + 1) % len(inputs)])):
                assert torch.equal(_bits(got), _bits(want)), f"eager call after replay {rep}, output {j}"


def _inputs(m, k, dtype, seed):
    return [rand_tokens(m, k, dtype, seed + i, n_outliers=4, outlier_scale=30.0).cuda() for i in range(3)]


@pytest.mark.parametrize("m,k,n,norm,dtype", [(16, 4096, 4096, "layernorm", "f16"),      # decode strip kernel
                                              (2, 4096, 3000, "rmsnorm", "bf16"),        # row GEMV
                                              (4, 1024, 17000, "none", "f16"),           # wide GEMV
                                              (300, 1024, 1000, "layernorm", "f32")],    # prefill tiles, ragged
                         ids=lambda v: str(v))
def test_graph_per_token_chain(m, k, n, norm, dtype):
    gamma, beta = _norm_params(k, norm, m + n)
    w = (rand_tokens(n, k, "f32", n + 1) * 0.02).to(DT[dtype]).cuda()
    absmax = sq.smoothquant_calibrate(rand_tokens(64, k, dtype, 7, n_outliers=4, outlier_scale=30.0).cuda(), norm,
                                      gamma, beta)
    f = sq.smoothquant_fold(absmax, w, 0.5, norm=norm, gamma=gamma, beta=beta)
    bias = (0.1 * torch.randn(n, generator=torch.Generator().manual_seed(3))).float().cuda()

    def make_outs():
        return (torch.empty(m, k, dtype=torch.int8, device="cuda"), torch.empty(m, device="cuda"),
                torch.empty(m, n, dtype=torch.float16, device="cuda"))

    def chain(x, outs):
        xq, xs, y = outs
        sq.sq_norm_quant(x, norm, f["gamma_f"], f["beta_f"], xq=xq, x_scale=xs)
        sq.sq_w8a8_gemm(xq, xs, f["wq"], f["w_scale"], bias, y=y)

    _check_graph(chain, make_outs, _inputs(m, k, dtype, 100 + m))


@pytest.mark.parametrize("mode", ["per_tensor", "static"])
def test_graph_per_tensor_chain(mode):
    m, k, n, norm = 40, 2048, 700, "rmsnorm"
    gamma, beta = _norm_params(k, norm, 5)
    w = (rand_tokens(n, k, "f32", 6) * 0.02).to(torch.bfloat16).cuda()
    absmax = sq.smoothquant_calibrate(rand_tokens(64, k, "bf16", 8, n_outliers=4, outlier_scale=30.0).cuda(), norm,
                                      gamma, beta)
    f = sq.smoothquant_fold_per_tensor(absmax, w, 0.5, norm=norm, gamma=gamma, beta=beta)
    step = sq.sq_static_step(absmax, f["s"])

    def make_outs():
        return (torch.empty(m, k, dtype=torch.int8, device="cuda"), torch.empty(m, device="cuda"),
                torch.empty(m, n, dtype=torch.bfloat16, device="cuda"))

    def chain(x, outs):
        xq, xs, y = outs
        if mode == "per_tensor":
            sq.sq_norm_quant_per_tensor(x, norm, f["gamma_f"], f["beta_f"], xq=xq, x_scale=xs)
        else:
            sq.sq_norm_quant_static(x, step, norm, f["gamma_f"], f["beta_f"], xq=xq, x_scale=xs)
        sq.sq_w8a8_gemm(xq, xs, f["wq"], f["w_scale"], out_dtype=torch.bfloat16, y=y)

    _check_graph(chain, make_outs, _inputs(m, k, "bf16", 200))


def test_graph_fp8_chain():
    m, k, n, norm = 64, 2048, 1000, "layernorm"
    gamma, beta = _norm_params(k, norm, 9)
    w = (rand_tokens(n, k, "f32", 10) * 0.02).to(torch.float16).cuda()
    absmax = sq.smoothquant_calibrate(rand_tokens(64, k, "f16", 11, n_outliers=4, outlier_scale=30.0).cuda(), norm,
                                      gamma, beta)
    f = sq.smoothquant_fold_fp8(absmax, w, 0.5, norm=norm, gamma=gamma, beta=beta)

    def make_outs():
        return (torch.empty(m, k, dtype=torch.uint8, device="cuda"), torch.empty(m, device="cuda"),
                torch.empty(m, n, dtype=torch.float32, device="cuda"))

    def chain(x, outs):
        xq, xs, y = outs
        sq.sq_norm_quant_fp8(x, norm, f["gamma_f"], f["beta_f"], xq=xq, x_scale=xs)
        sq.sq_fp8_gemm(xq, xs, f["wq"], f["w_scale"], out_dtype=torch.float32, y=y)

    _check_graph(chain, make_outs, _inputs(m, k, "f16", 300))


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_graph_llm_int8(noalloc):
    m, k, n, norm = 48, 1024, 700, "layernorm"
    gamma, beta = _norm_params(k, norm, 12)
    w = (rand_tokens(n, k, "f32", 13) * 0.02).to(torch.float16).cuda()
    wq, ws = sq.sq_norm_quant(w, "none")
    workspace = torch.empty(sq.sq_llm_int8_workspace(m, n, k)["total"], dtype=torch.uint8, device="cuda")

    def make_outs():
        return (torch.empty(m, n, dtype=torch.float16, device="cuda"),)

    def chain(x, outs):
        if noalloc:
            sq.sq_llm_int8_linear_noalloc(x, w, wq, ws, norm, gamma, beta, 1e-5, 6.0, y=outs[0])
        else:
            sq.sq_llm_int8_linear(x, w, wq, ws, norm, gamma, beta, 1e-5, 6.0, y=outs[0], workspace=workspace)

    _check_graph(chain, make_outs, _inputs(m, k, "f16", 400))
