"""The GPU checks' own tie handling, exercised on the CPU with outputs built from the oracle.

On a row whose mean sits exactly on a binary32 midpoint both roundings of the
mean are correct. A check must accept the codes of either rounding and reject
codes that are neither (here: the codes of one rounding with a wrong sign).
"""
import numpy as np
import pytest

import oracle as O
from tests.gpu_check import check_norm_quant
from tests.test_gpu_granularity import _compare

F32 = np.float32


def _tie_row():
    # mean 1 + 2^-24: exactly the midpoint of the binary32 neighbours 1 and 1 + 2^-23
    return np.array([[1.0] * 32 + [1.0 + 2.0 ** -23] * 32], F32)


@pytest.mark.parametrize("fp8", [False, True])
def test_per_tensor_compare_accepts_either_rounding_and_nothing_else(fp8):
    x = _tie_row()
    nq = O.norm_quant_fp8_per_tensor if fp8 else O.norm_quant_per_tensor
    quant = O.quantize_tensor_fp8 if fp8 else O.quantize_tensor
    q, xs, info = nq(x, "f32", O.LAYERNORM)
    assert info["near_tie"][0]
    src = (x, "f32", O.LAYERNORM, None, None, 1e-5)
    alts = [quant(y, step=xs[0])[0] for y in O.row_y_variants(x[0], "f32", O.LAYERNORM)]
    other = next(a for a in alts if not np.array_equal(a, q))
    assert _compare(q, xs, info, q, xs, "own", src, fp8) == 0
    assert _compare(q, xs, info, other, xs, "other", src, fp8) == 1
    wrong = (other.astype(np.int16) ^ 0x80).astype(q.dtype) if fp8 else (-other.astype(np.int16)).astype(np.int8)
    assert not any(np.array_equal(wrong, a) for a in alts)
    with pytest.raises(AssertionError):
        _compare(q, xs, info, wrong, xs, "wrong", src, fp8)


def test_per_row_check_accepts_either_rounding_and_nothing_else():
    x = _tie_row()
    variants = O.norm_quant_row_variants(x[0], "f32", O.LAYERNORM)
    assert len(variants) == 2
    for vq, vs in variants:
        assert check_norm_quant(x, "f32", O.LAYERNORM, None, None, 1e-5, vq, vs) in (0, 1)
    vq, vs = variants[1]
    with pytest.raises(AssertionError):
        check_norm_quant(x, "f32", O.LAYERNORM, None, None, 1e-5, (-vq.astype(np.int16)).astype(np.int8), vs)
