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


def _llm_parts(d, count, torch_half):
    """What a correct GPU call would leave in its workspace, built from the oracle (CPU tensors)."""
    import torch
    import oracle.llm_int8 as L
    p = (count + 31) // 32 * 32
    m, n = d["xq"].shape[0], d["wo"].shape[0]

    def pad(v):
        out = np.zeros((v.shape[0], p), F32)
        out[:, :count] = v
        if torch_half == torch.bfloat16:
            return torch.from_numpy(O.f32_to_bf16_bits(out).view(np.int16)).view(torch.bfloat16)
        return torch.from_numpy(out.astype(np.float16))
    y32 = (d["deq"] + d["acc16"].astype(F32)).astype(F32)
    return {"count": count, "idx": torch.from_numpy(d["O"].astype(np.int32)),
            "xq": torch.from_numpy(d["xq"]), "x_scale": torch.from_numpy(d["x_scale"]),
            "x16": pad(d["xo"]), "w16": pad(d["wo"]), "deq": torch.from_numpy(d["deq"])}, y32, m, n, L


@pytest.mark.parametrize("wdt", ["f16", "bf16"])
def test_llm_int8_check_accepts_a_correct_evaluation_and_rejects_slips(wdt):
    import torch
    from tests.gpu_check import check_llm_int8
    rng = np.random.default_rng(21)
    x = rng.standard_normal((12, 128)).astype(F32)
    x[:, [5, 90, 91]] *= 20
    w32 = (rng.standard_normal((40, 128)) * 0.05).astype(F32)
    w = O.f32_to_bf16_bits(w32) if wdt == "bf16" else w32.astype(np.float16)
    import oracle.llm_int8 as L
    d = L.decompose(x, "f32", O.NONE, w, w_dtype=wdt, out_dtype="f32")
    assert d["O"].tolist() == [5, 90, 91]
    half = torch.bfloat16 if wdt == "bf16" else torch.float16
    parts, y32, _, _, _ = _llm_parts(d, 3, half)
    check_llm_int8(x, "f32", O.NONE, None, None, 1e-5, 6.0, w, wdt, "f32", parts, y32)
    for key, slip in (("x16", lambda t: t.clone().view(torch.int16).add_(1).view(half)),
                      ("deq", lambda t: t.clone().view(torch.int32).add_(1).view(torch.float32)),
                      ("xq", lambda t: t.clone().add_(1))):
        bad = dict(parts, **{key: slip(parts[key])})
        with pytest.raises(AssertionError):
            check_llm_int8(x, "f32", O.NONE, None, None, 1e-5, 6.0, w, wdt, "f32", bad, y32)
    with pytest.raises(AssertionError):                             # an output far outside the bound
        check_llm_int8(x, "f32", O.NONE, None, None, 1e-5, 6.0, w, wdt, "f32", parts, y32 * np.float32(1.001))
