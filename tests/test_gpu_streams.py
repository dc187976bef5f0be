"""Re-entrancy of the library (needs an MI355X): the whole chain issued from two host threads on two
streams at once (ctypes releases the GIL during each call) gives bit for bit what a serial run on
the default stream gives. The library keeps no state, so nothing may leak between the two."""
import threading

import pytest
import torch

import w8a8_int8_linear_amd as sq
from synth import site_inputs

pytestmark = pytest.mark.gpu


def chain(inp, fp8=False):
    x, xc, w, g, b = inp["x"], inp["x_cal"], inp["w"], inp["gamma"], inp["beta"]
    amax = sq.smoothquant_calibrate(xc, "layernorm", g, b, 1e-5)
    if fp8:
        fo = sq.smoothquant_fold_fp8(amax, w, 0.5, 1e-5, "layernorm", g, b)
        xq, xs = sq.sq_norm_quant_fp8(x, "layernorm", fo["gamma_f"], fo["beta_f"], 1e-5)
        y = sq.sq_fp8_gemm(xq, xs, fo["wq"], fo["w_scale"], out_dtype=torch.float16)
    else:
        fo = sq.smoothquant_fold(amax, w, 0.5, 1e-5, "layernorm", g, b)
        xq, xs = sq.sq_norm_quant(x, "layernorm", fo["gamma_f"], fo["beta_f"], 1e-5)
        y = sq.sq_w8a8_gemm(xq, xs, fo["wq"], fo["w_scale"], out_dtype=torch.float16)
    return [amax, fo["s"], fo["wq"], fo["w_scale"], xq, xs, y]


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
def test_two_threads_two_streams_match_serial(fp8):
    # two different problems: an OPT-6.7B prefill site (M 256) and an OPT-66B decode site (M 32)
    inputs = [site_inputs(2, 0, m=256, device="cuda", w_rows=4096), site_inputs(3, 1, m=32, device="cuda", w_rows=9216)]
    torch.cuda.synchronize()
    serial = [chain(inp, fp8) for inp in inputs]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results, errors = [None, None], []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):                       # several rounds, so the two streams overlap
                    results[i] = chain(inputs[i], fp8)
            streams[i].synchronize()
        except Exception as e:                           # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for a, b in zip(serial[i], results[i]):
            assert torch.equal(a, b)
