"""Workload definitions and seeded generators (random draws and dtype casts only).

The workloads stand in for the real models and calibration sets that the
SmoothQuant pages measure on (OPT, LLaMA-2, MT-NLG layers calibrated on a few
hundred sentences): they reproduce the layer shapes and the activation
structure the pages describe -- a handful of persistent outlier channels that
are tens of times larger than the rest in every token ("LLM.int8() and
SmoothQuant", section "The problem: activations, not weights"; "SmoothQuant, in
depth", section "The problem SmoothQuant solves").

Every tensor is drawn from a torch generator seeded from (workload, site,
stream), on the device the caller names. The same seed gives the same values on
the same device kind; CPU and GPU draws differ, so GPU tests copy their inputs
back to the host before handing them to the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Site:
    """One norm (or none) feeding one or more projections that share a smoothing vector.

    ``parts`` lists the projections concatenated along the output dimension
    (q/k/v or gate/up); ``n`` is their total output width.
    """
    name: str
    norm: str                 # "none" | "layernorm" | "rmsnorm"
    k: int
    parts: tuple              # ((name, n_out), ...)
    n_outliers: int
    outlier_scale: float
    w_sigma: float

    @property
    def n(self) -> int:
        return sum(p[1] for p in self.parts)


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    dtype: str                # activation and weight storage dtype
    out_dtype: str            # GEMM output dtype
    m: tuple                  # runtime token counts
    m_cal: int                # calibration tokens per site
    alpha: float
    act_dist: str             # "normal" | "student_t4"
    sites: tuple = field(default_factory=tuple)


WORKLOADS = {
    1: Workload(
        1, "tiny_linear_m16_k512_n512", "f32", "f32", (16,), 64, 0.5, "normal",
        (Site("x->linear", "none", 512, (("linear", 512),), 4, 50.0, 0.02),)),
    2: Workload(
        2, "opt6.7b_prefill_m2048_h4096", "f16", "f16", (2048,), 512, 0.5, "normal",
        (Site("ln1->qkv", "layernorm", 4096, (("qkv", 12288),), 4, 60.0, 0.02),
         Site("ln2->fc1", "layernorm", 4096, (("fc1", 16384),), 4, 60.0, 0.02))),
    3: Workload(
        3, "opt66b_decode_h9216", "f16", "f16", (1, 8, 32, 64), 512, 0.5, "normal",
        (Site("ln->proj9216", "layernorm", 9216, (("proj", 9216),), 6, 40.0, 0.02),
         Site("ln->fc1", "layernorm", 9216, (("fc1", 36864),), 6, 40.0, 0.02))),
    4: Workload(
        4, "llama2_7b_block_m4096_h4096", "bf16", "bf16", (4096,), 512, 0.8, "student_t4",
        (Site("rms1->qkv", "rmsnorm", 4096, (("q", 4096), ("k", 4096), ("v", 4096)), 8, 80.0, 0.02),
         Site("rms2->gate_up", "rmsnorm", 4096, (("gate", 11008), ("up", 11008)), 8, 80.0, 0.02))),
    5: Workload(
        5, "mtnlg530b_width_m8192_h20480", "f16", "f16", (8192,), 512, 0.5, "normal",
        (Site("ln->fc1", "layernorm", 20480, (("fc1", 81920),), 10, 100.0, 0.01),
         Site("act->fc2", "none", 81920, (("fc2", 20480),), 41, 100.0, 0.01))),
}

_STREAMS = {"outliers": 1, "tokens": 2, "calib": 3, "weights": 4, "gamma": 5, "beta": 6}


def _seed(wl_id: int, site_idx: int, stream: str, sub: int = 0) -> int:
    return (wl_id << 40) | (site_idx << 32) | (_STREAMS[stream] << 24) | sub


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def outlier_channels(wl: Workload, site_idx: int) -> np.ndarray:
    """Sorted indices of the persistent outlier channels (same in every token)."""
    site = wl.sites[site_idx]
    g = _gen(_seed(wl.id, site_idx, "outliers"), "cpu")
    idx = torch.randperm(site.k, generator=g)[: site.n_outliers]
    return np.sort(idx.numpy())


def _activations(wl: Workload, site_idx: int, m: int, stream: str, device, sub: int = 0):
    site = wl.sites[site_idx]
    g = _gen(_seed(wl.id, site_idx, stream, sub), device)
    if wl.act_dist == "normal":
        x = torch.randn(m, site.k, generator=g, device=device, dtype=torch.float32)
    elif wl.act_dist == "student_t4":
        # Student-t with 4 degrees of freedom: Z / sqrt(chi2_4 / 4), chi2_4 = 2 (E1 + E2).
        z = torch.randn(m, site.k, generator=g, device=device, dtype=torch.float32)
        u = torch.rand(2, m, site.k, generator=g, device=device, dtype=torch.float32)
        e = -torch.log1p(-u)            # Exp(1) draws, finite since u < 1
        x = z / torch.sqrt((e[0] + e[1]) * 0.5)
        del z, u, e
    else:
        raise ValueError(wl.act_dist)
    cols = torch.from_numpy(outlier_channels(wl, site_idx)).to(device)
    if cols.numel():
        x[:, cols] *= site.outlier_scale
    return x.to(DTYPES[wl.dtype])


def token_block(wl: Workload, site_idx: int, m: int, device="cpu", sub: int = 0) -> torch.Tensor:
    """Runtime tokens ``[m, K]`` entering the site (storage dtype of the workload)."""
    return _activations(wl, site_idx, m, "tokens", device, sub)


def calibration_block(wl: Workload, site_idx: int, device="cpu") -> torch.Tensor:
    """Calibration tokens ``[m_cal, K]`` drawn from the same distribution."""
    return _activations(wl, site_idx, wl.m_cal, "calib", device)


def weight_block(wl: Workload, site_idx: int, device="cpu", rows: int | None = None) -> torch.Tensor:
    """Concatenated projection weights ``[N, K]`` (torch Linear layout), sigma as stated.

    ``rows`` draws only that many output channels of the first projection (a
    smaller sample with the same distribution, for host-side baselines).
    """
    site = wl.sites[site_idx]
    parts = []
    for j, (_, n_out) in enumerate(site.parts):
        if rows is not None:
            n_out = rows
        g = _gen(_seed(wl.id, site_idx, "weights", j), device)
        w = torch.randn(n_out, site.k, generator=g, device=device, dtype=torch.float32)
        w *= site.w_sigma
        parts.append(w.to(DTYPES[wl.dtype]))
        del w
        if rows is not None:
            break
    return parts[0] if len(parts) == 1 else torch.cat(parts, dim=0)


def norm_params(wl: Workload, site_idx: int, device="cpu"):
    """(gamma, beta) fp32 ``[K]`` of the norm in front of the site; None where absent."""
    site = wl.sites[site_idx]
    if site.norm == "none":
        return None, None
    g = _gen(_seed(wl.id, site_idx, "gamma"), device)
    gamma = 1.0 + 0.1 * torch.randn(site.k, generator=g, device=device, dtype=torch.float32)
    beta = None
    if site.norm == "layernorm":
        g = _gen(_seed(wl.id, site_idx, "beta"), device)
        beta = 0.1 * torch.randn(site.k, generator=g, device=device, dtype=torch.float32)
    return gamma, beta


def site_inputs(wl_id: int, site_idx: int, m: int | None = None, device="cpu", w_rows: int | None = None) -> dict:
    """Everything one site needs: runtime tokens, calibration tokens, weights, norm params."""
    wl = WORKLOADS[wl_id]
    site = wl.sites[site_idx]
    m = wl.m[0] if m is None else m
    gamma, beta = norm_params(wl, site_idx, device)
    return {
        "workload": wl, "site": site, "x": token_block(wl, site_idx, m, device),
        "x_cal": calibration_block(wl, site_idx, device), "w": weight_block(wl, site_idx, device, w_rows),
        "gamma": gamma, "beta": beta, "outliers": outlier_channels(wl, site_idx),
    }


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy for the oracle: fp32/fp16 as themselves, bf16 as its uint16 bit pattern."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ----------------------------------------------------------------------------- ad-hoc seeded tensors

def rand_tokens(m: int, k: int, dtype: str, seed: int, n_outliers: int = 0, outlier_scale: float = 50.0,
                dist: str = "normal", mean: float = 0.0, scale: float = 1.0) -> torch.Tensor:
    """[m, k] activations on the CPU: N(mean, scale) (or Student-t(4)) with optional persistent outliers."""
    g = _gen(seed, "cpu")
    x = torch.randn(m, k, generator=g, dtype=torch.float32)
    if dist == "student_t4":
        u = torch.rand(2, m, k, generator=g, dtype=torch.float32)
        e = -torch.log1p(-u)
        x = x / torch.sqrt((e[0] + e[1]) * 0.5)
    x = x * scale + mean
    if n_outliers:
        cols = torch.randperm(k, generator=g)[:n_outliers]
        x[:, cols] *= outlier_scale
    return x.to(DTYPES[dtype])


def rand_int8(shape, seed: int, lo: int = -127, hi: int = 127) -> torch.Tensor:
    """Uniform int8 codes in [lo, hi] on the CPU."""
    g = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, dtype=torch.int16).to(torch.int8)


def rand_positive(n: int, seed: int, lo: float = 1e-3, hi: float = 1.0) -> torch.Tensor:
    """n fp32 values log-uniform in [lo, hi] (per-row / per-channel INT8 steps)."""
    g = _gen(seed, "cpu")
    u = torch.rand(n, generator=g, dtype=torch.float64)
    return torch.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).to(torch.float32)
