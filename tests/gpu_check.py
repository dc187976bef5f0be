"""Comparison helpers for the GPU parity tests: the HIP results against the oracle.

Integer codes, steps and accumulators must match bit for bit. Where the oracle
reports a near-tie (a norm statistic or a smoothing factor whose exact value
lies within a tiny distance of a binary32 rounding boundary), either neighbour
is a correct rounding: the check accepts the GPU's choice only if it is one of
the two candidates the oracle computed, and continues with that candidate.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from synth import to_numpy

F32 = np.float32


def bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16) if a.dtype.itemsize == 2 else a


def host(t: torch.Tensor) -> np.ndarray:
    return to_numpy(t)


def check_norm_quant(x_np, dtype, norm, gamma_f, beta_f, eps, xq_gpu, xs_gpu, label=""):
    """Codes and steps of every row bit-exact; near-tie rows may take either statistic rounding."""
    q, step, info = O.norm_quant(x_np, dtype, norm, gamma_f, beta_f, eps)
    xq_gpu = np.asarray(xq_gpu)
    xs_gpu = np.asarray(xs_gpu, F32)
    bad = np.where((q != xq_gpu).any(axis=1) | (bits(step) != bits(xs_gpu)))[0]
    ties = 0
    for r in bad:
        assert info["near_tie"][r], (
            f"{label}: row {r} differs (step {step[r]!r} vs {xs_gpu[r]!r}, "
            f"{int((q[r] != xq_gpu[r]).sum())} codes)")
        variants = O.norm_quant_row_variants(x_np[r], dtype, norm, gamma_f, beta_f, eps)
        assert any(np.array_equal(vq[0], xq_gpu[r]) and bits(vs)[0] == bits(xs_gpu[r:r + 1])[0]
                   for vq, vs in variants), f"{label}: near-tie row {r} matches no correct rounding"
        ties += 1
    return ties


def check_calibrate(x_np, dtype, norm, gamma, beta, eps, amax_gpu, prior=None, label=""):
    a, info = O.calibrate(x_np, dtype, norm, gamma, beta, eps, absmax=prior)
    amax_gpu = np.asarray(amax_gpu, F32)
    diff = bits(a) != bits(amax_gpu)
    if diff.any():
        # a channel may take its max from a near-tie row evaluated with the other statistic rounding
        tie_rows = np.where(info["near_tie"])[0]
        assert len(tie_rows), f"{label}: {int(diff.sum())} channels differ with no near-tie row"
        cands = [a]
        for r in tie_rows:
            st = info["alt"][r]
            for mu in {float(st["mu"]), float(st["mu_other"])}:
                for var in {float(st["var"]), float(st["var_other"])}:
                    y = O.normalize(O.widen(x_np[r:r + 1], dtype), norm, [mu], [var], gamma, beta, eps)
                    cands.append(np.abs(y[0]).astype(F32))
        ok = np.any(bits(np.stack(cands)) == bits(amax_gpu)[None, :], axis=0)
        assert ok[diff].all(), f"{label}: channels {np.where(diff & ~ok)[0][:8]} differ"
    return a


def check_fold(a_ref, w_np, dtype, alpha, eps, norm, gamma, beta, out_gpu, rows=None, label=""):
    """s, gamma', beta' over all channels; codes and steps of W rows `rows` (all rows by default).

    out_gpu holds the HIP results; with `rows`, out_gpu["wq"] / ["w_scale"] may be
    just those rows (already gathered on the device).
    """
    s_ref, dist, other = O.smoothing_factors(a_ref, O.weight_colmax(w_np, dtype), alpha, eps)
    s_gpu = host(out_gpu["s"])
    diff = bits(s_ref) != bits(s_gpu)
    if diff.any():
        tie = dist < O.smoothquant_oracle.NEAR_TIE
        other_ok = bits(other) == bits(s_gpu)
        assert (tie & other_ok)[diff].all(), f"{label}: s differs at {np.where(diff & ~(tie & other_ok))[0][:8]}"
        s_ref = np.where(diff, other, s_ref)
    w_sel = w_np if rows is None else w_np[rows]
    f = O.fold(a_ref, w_sel, dtype, alpha, eps, norm, gamma, beta, s=s_ref)
    assert np.array_equal(bits(f["gamma_f"]), bits(host(out_gpu["gamma_f"]))), f"{label}: gamma' differs"
    if f["beta_f"] is not None:
        assert np.array_equal(bits(f["beta_f"]), bits(host(out_gpu["beta_f"]))), f"{label}: beta' differs"
    wq_gpu = host(out_gpu["wq"])
    ws_gpu = host(out_gpu["w_scale"])
    if rows is not None and wq_gpu.shape[0] != len(rows):
        wq_gpu, ws_gpu = wq_gpu[rows], ws_gpu[rows]
    bad_rows = np.where((f["wq"] != wq_gpu).any(axis=1))[0]
    assert not len(bad_rows), f"{label}: weight codes differ in rows {bad_rows[:8]}"
    assert np.array_equal(bits(f["w_scale"]), bits(ws_gpu)), f"{label}: w_scale differs"
    return f, int(diff.sum())


def check_output(y_gpu_np, out_ref, v32_ref, out_dtype, label=""):
    """Output within 2e-3 relative of the oracle's output in the same output type, and
    (the epilogue order being pinned) bit-identical to it.

    The bound is taken after both sides convert to the output type: bfloat16 keeps
    8 significant bits, so its own rounding may move a value by up to 2^-8 of it,
    more than 2e-3, while fp16 (2^-11) and fp32 stay well inside.
    """
    def as_f64(a):
        a = np.ascontiguousarray(a)
        if out_dtype == "bf16":
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)
    y, ref = as_f64(y_gpu_np), as_f64(out_ref)
    half_ulp_min = {"f32": 2.0 ** -150, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}[out_dtype]
    err = np.abs(y - ref)
    assert np.all(err <= 2e-3 * np.abs(ref) + half_ulp_min), (
        f"{label}: max rel err {np.max(err / np.maximum(np.abs(ref), 1e-30)):.3g}")
    u = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[out_dtype]
    assert np.all(np.abs(ref - v32_ref.astype(np.float64)) <= u * np.abs(v32_ref.astype(np.float64)) + half_ulp_min)
    exact = np.mean(bits(np.ascontiguousarray(y_gpu_np)) == bits(np.ascontiguousarray(out_ref)))
    assert exact == 1.0, f"{label}: {100 * (1 - exact):.4f}% of outputs not bit-identical"


def _vals16(t, fmt):
    """A device tensor of fp16 / bf16 numbers as binary32 values (host() gives bf16 as bit patterns)."""
    a = host(t)
    return O.widen(a, "bf16") if fmt == "bf16" else a.astype(F32)


def _f16_bits(v32, fmt):
    """Bit patterns of binary32 values that are fp16 / bf16 numbers."""
    v32 = np.asarray(v32, F32)
    return v32.astype(np.float16).view(np.uint16) if fmt == "f16" else O.f32_to_bf16_bits(v32)


def check_llm_int8(x_np, dtype, norm, gamma, beta, eps, tau, w_np, w_dtype, out_dtype, parts, y_gpu, bias=None,
                   outliers=None, label=""):
    """The LLM.int8() decomposition on the GPU against oracle.llm_int8, part by part.

    x_np holds the rows being checked (all of them, or a sample with `outliers` = the set the whole
    batch gave); w_np all weight rows, or a sample of them (parts["deq"], parts["w16"] and y_gpu then
    hold just those columns / rows). Integer and 16-bit parts are bit-exact: the outlier set (when x_np
    is the whole batch), the INT8 codes and steps, the 16-bit operands, deq. A row whose statistics are a near-tie may take either rounding
    (codes, step and 16-bit values of one of the oracle's candidate y rows). The output must lie within
    output_bound of deq + the exact 16-bit product, both taken from the accepted parts.
    """
    import oracle.llm_int8 as L
    count = parts["count"]
    o_gpu = host(parts["idx"]).astype(np.int64)
    assert len(o_gpu) == count and np.all(np.diff(o_gpu) > 0), f"{label}: outlier list not ascending"
    d = L.decompose(x_np, dtype, norm, w_np, gamma, beta, eps, tau, w_dtype, bias=bias, out_dtype=out_dtype,
                    outliers=o_gpu if outliers is None else outliers)
    if outliers is None:
        o_ref = L.outlier_channels(d["y"], tau)
        if not np.array_equal(o_ref, o_gpu):
            # only a near-tie row, normalised with its other statistic rounding, may move a channel across tau
            assert d["near_tie"].any(), f"{label}: outliers {o_gpu[:8]} vs oracle {o_ref[:8]}"
    else:
        assert np.array_equal(np.asarray(outliers), o_gpu), f"{label}: outlier set differs"
    o = d["O"]
    fmt = d["fmt"]
    p = (count + 31) // 32 * 32
    xq_gpu, xs_gpu = host(parts["xq"]), host(parts["x_scale"])
    x16_gpu = _vals16(parts["x16"], fmt)
    assert x16_gpu.shape[1] == p and not x16_gpu[:, count:].any(), f"{label}: 16-bit padding not zero"
    x16_bits = _f16_bits(x16_gpu[:, :count], fmt)
    bad = np.where((xq_gpu != d["xq"]).any(axis=1) | (bits(xs_gpu) != bits(d["x_scale"]))
                   | (x16_bits != _f16_bits(d["xo"], fmt)).any(axis=1))[0]
    for r in bad:
        assert d["near_tie"][r], f"{label}: row {r} differs (step {d['x_scale'][r]!r} vs {xs_gpu[r]!r})"
        ok = False
        for y in O.row_y_variants(x_np[r], dtype, norm, gamma, beta, eps):
            yi = y.copy()
            yi[:, o] = 0
            q, s = O.quantize_rows(yi)
            ok |= (np.array_equal(q[0], xq_gpu[r]) and bits(s)[0] == bits(xs_gpu[r:r + 1])[0]
                   and np.array_equal(_f16_bits(L.round16(y[0, o], fmt), fmt), x16_bits[r]))
        assert ok, f"{label}: near-tie row {r} matches no correct rounding"
    w16_gpu = _vals16(parts["w16"], fmt)
    assert w16_gpu.shape[1] == p and not w16_gpu[:, count:].any()
    assert np.array_equal(_f16_bits(w16_gpu[:, :count], fmt), _f16_bits(d["wo"], fmt)), f"{label}: w16 differs"
    _, deq = O.dequantize(O.int_gemm(xq_gpu, d["wq"]), xs_gpu, d["w_scale"])
    deq_gpu = host(parts["deq"])
    assert np.array_equal(bits(deq), bits(deq_gpu)), f"{label}: deq differs in {int((bits(deq) != bits(deq_gpu)).sum())}"
    # the output, from the accepted parts
    d2 = dict(d, deq=deq, xo=x16_gpu[:, :count])
    d2["acc16"] = L.gemm16(d2["xo"], d["wo"])
    d2["sum_abs16"] = L.gemm16(np.abs(d2["xo"]), np.abs(d["wo"]))
    d2["ref"] = deq.astype(np.float64) + d2["acc16"] + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :])
    y = np.ascontiguousarray(np.asarray(y_gpu))
    y64 = (y.astype(np.uint32) << 16).view(F32).astype(np.float64) if out_dtype == "bf16" else y.astype(np.float64)
    err = np.abs(y64 - d2["ref"])
    bound = L.output_bound(d2, n_pad=p)
    worst = np.max(err / np.maximum(bound, 1e-300)) if err.size else 0.0
    assert np.all(err <= bound), f"{label}: output outside the bound (worst {worst:.3g} of it)"
    return d2, worst
