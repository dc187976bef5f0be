"""sq_llm_int8_linear_noalloc through the C ABI (needs an MI355X): two calls in a row, the second
smaller, each bit for bit equal to sq_llm_int8_linear with a workspace of its own; and a shape whose
workspace exceeds the fixed scratch is refused before anything is launched."""
import pytest
import torch

import w8a8_int8_linear_amd as sq
from synth import rand_tokens

pytestmark = pytest.mark.gpu


def _case(m, k, n, seed, norm, dtype):
    x = rand_tokens(m, k, dtype, seed, n_outliers=5, outlier_scale=40.0).cuda()
    w = (rand_tokens(n, k, "f32", seed + 1) * 0.02).to(x.dtype).cuda()
    g = torch.Generator().manual_seed(seed + 2)
    gamma = (1 + 0.1 * torch.randn(k, generator=g)).float().cuda() if norm != "none" else None
    beta = (0.1 * torch.randn(k, generator=g)).float().cuda() if norm == "layernorm" else None
    wq, ws = sq.sq_norm_quant(w, "none")
    return x, w, wq, ws, gamma, beta


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    for m, k, n, seed, norm, dtype, out in [(300, 2048, 3000, 11, "layernorm", "f16", torch.float16),
                                            (24, 1024, 700, 12, "rmsnorm", "bf16", torch.bfloat16)]:
        x, w, wq, ws, gamma, beta = _case(m, k, n, seed, norm, dtype)
        need = sq.sq_llm_int8_workspace(m, n, k)["total"]
        assert need <= sq.SQ_NOALLOC_SCRATCH_BYTES
        y0 = sq.sq_llm_int8_linear_noalloc(x, w, wq, ws, norm, gamma, beta, 1e-5, 6.0, out_dtype=out)
        y1, _ = sq.sq_llm_int8_linear(x, w, wq, ws, norm, gamma, beta, 1e-5, 6.0, out_dtype=out)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), f"{m}x{k}x{n}"


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    m, k, n = 64, 9216, 9216
    assert sq.sq_llm_int8_workspace(m, n, k)["total"] > sq.SQ_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(m, k, dtype=torch.float16, device="cuda")
    w = torch.zeros(n, k, dtype=torch.float16, device="cuda")
    wq = torch.zeros(n, k, dtype=torch.int8, device="cuda")
    ws = torch.zeros(n, dtype=torch.float32, device="cuda")
    y = torch.full((m, n), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(sq.SmoothQuantError) as e:
        sq.sq_llm_int8_linear_noalloc(x, w, wq, ws, "none", out_dtype=torch.float16, y=y)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert (y == 7.0).all()                                   # nothing was launched
