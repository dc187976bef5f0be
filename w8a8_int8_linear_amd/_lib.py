"""ctypes binding of libsmoothquant.so (argument marshalling only).

Each wrapper takes torch tensors for their device memory and the current HIP
stream, checks shapes and dtypes, and calls the C entry point of the same
name. Every computation runs in the library's HIP kernels; there is no
fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmoothquant.so")

SQ_OK = 0
SQ_DT_F32, SQ_DT_F16, SQ_DT_BF16, SQ_DT_I32 = 0, 1, 2, 3
SQ_NORM_NONE, SQ_NORM_LAYERNORM, SQ_NORM_RMSNORM = 0, 1, 2
SQ_K_MAX = 133120

_DT = {torch.float32: SQ_DT_F32, torch.float16: SQ_DT_F16, torch.bfloat16: SQ_DT_BF16, torch.int32: SQ_DT_I32}
_NORM = {"none": SQ_NORM_NONE, "layernorm": SQ_NORM_LAYERNORM, "rmsnorm": SQ_NORM_RMSNORM,
         SQ_NORM_NONE: SQ_NORM_NONE, SQ_NORM_LAYERNORM: SQ_NORM_LAYERNORM, SQ_NORM_RMSNORM: SQ_NORM_RMSNORM}

EXPORTS = ("smoothquant_calibrate", "smoothquant_fold", "sq_norm_quant", "sq_w8a8_gemm",
           "sq_norm_quant_per_tensor", "sq_norm_quant_static", "sq_static_step", "smoothquant_fold_per_tensor",
           "sq_norm_quant_fp8", "smoothquant_fold_fp8", "sq_fp8_gemm", "sq_norm_quant_fp8_per_tensor",
           "sq_norm_quant_fp8_static", "sq_static_step_fp8", "smoothquant_fold_fp8_per_tensor",
           "sq_llm_int8_workspace", "sq_llm_int8_linear", "sq_llm_int8_linear_noalloc", "sq_status_string")
SQ_NOALLOC_SCRATCH_BYTES = 134217728
SQ_ERR_TOO_LARGE = 8

LLM_INT8_FIELDS = ("total", "count", "idx", "absmax", "gamma_m", "beta_m", "stats", "xq", "x_scale", "x16", "w16",
                   "deq")


class _LlmLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_uint64) for name in LLM_INT8_FIELDS]


class SmoothQuantError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python w8a8_int8_linear_amd/build.py` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I64, F, D, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_int
    lib.smoothquant_calibrate.argtypes = [P, I, I64, I64, I, P, P, F, P, P]
    lib.smoothquant_fold.argtypes = [P, P, I, I64, I64, D, F, I, P, P, P, P, P, P, P, P]
    lib.sq_norm_quant.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P]
    lib.sq_w8a8_gemm.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P]
    lib.sq_norm_quant_per_tensor.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P]
    lib.sq_norm_quant_static.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P, P]
    lib.sq_static_step.argtypes = [P, P, I64, P, P]
    lib.smoothquant_fold_per_tensor.argtypes = [P, P, I, I64, I64, D, F, I, P, P, P, P, P, P, P, P]
    lib.sq_norm_quant_fp8.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P]
    lib.smoothquant_fold_fp8.argtypes = [P, P, I, I64, I64, D, F, I, P, P, P, P, P, P, P, P]
    lib.sq_fp8_gemm.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P]
    lib.sq_norm_quant_fp8_per_tensor.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P]
    lib.sq_norm_quant_fp8_static.argtypes = [P, I, I64, I64, I, P, P, F, P, P, P, P]
    lib.sq_static_step_fp8.argtypes = [P, P, I64, P, P]
    lib.smoothquant_fold_fp8_per_tensor.argtypes = [P, P, I, I64, I64, D, F, I, P, P, P, P, P, P, P, P]
    lib.sq_llm_int8_workspace.argtypes = [I64, I64, I64, ctypes.POINTER(_LlmLayout)]
    lib.sq_llm_int8_linear.argtypes = [P, I, I64, I64, I, P, P, F, F, P, I, P, P, I64, P, P, I, P, ctypes.c_uint64, P]
    lib.sq_llm_int8_linear_noalloc.argtypes = [P, I, I64, I64, I, P, P, F, F, P, I, P, P, I64, P, P, I, P]
    lib.sq_status_string.argtypes = [I]
    lib.sq_status_string.restype = ctypes.c_char_p
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = I
    return lib


lib = load_library()


def status_string(status: int) -> str:
    return lib.sq_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _check(fn: str, status: int):
    if status != SQ_OK:
        raise SmoothQuantError(fn, status)


_ACT = (torch.float32, torch.float16, torch.bfloat16)


def smoothquant_calibrate(x, norm="none", gamma=None, beta=None, eps=1e-5, absmax=None):
    """Running per-channel max of |norm(x)| into absmax [K] fp32 (created zeroed if None)."""
    _dev(x, "x", _ACT)
    m, k = x.shape
    if absmax is None:
        absmax = torch.zeros(k, dtype=torch.float32, device=x.device)
    _dev(absmax, "absmax", torch.float32, (k,))
    _dev(gamma, "gamma", torch.float32, (k,))
    _dev(beta, "beta", torch.float32, (k,))
    with torch.cuda.device(x.device):
        _check("smoothquant_calibrate", lib.smoothquant_calibrate(
            _ptr(x), _DT[x.dtype], m, k, _NORM[norm], _ptr(gamma), _ptr(beta), eps, _ptr(absmax), _stream(x)))
    return absmax


def smoothquant_fold(act_absmax, w, alpha, eps=1e-5, norm="none", gamma=None, beta=None, out=None):
    """Smoothing factors, folded norm parameters and INT8 weights for w [N, K] (one step per output row).

    Returns dict(s, gamma_f, beta_f, wq, w_scale); `out` may supply those buffers.
    """
    return _fold("smoothquant_fold", act_absmax, w, alpha, eps, norm, gamma, beta, out)


def smoothquant_fold_fp8(act_absmax, w, alpha, eps=1e-5, norm="none", gamma=None, beta=None, out=None):
    """As smoothquant_fold with FP8 (OCP E4M3) weight codes (wq uint8) and steps absmax / 448."""
    return _fold("smoothquant_fold_fp8", act_absmax, w, alpha, eps, norm, gamma, beta, out)


def smoothquant_fold_per_tensor(act_absmax, w, alpha, eps=1e-5, norm="none", gamma=None, beta=None, out=None):
    """As smoothquant_fold with one weight step for the whole tensor (w_scale holds it repeated)."""
    return _fold("smoothquant_fold_per_tensor", act_absmax, w, alpha, eps, norm, gamma, beta, out)


def smoothquant_fold_fp8_per_tensor(act_absmax, w, alpha, eps=1e-5, norm="none", gamma=None, beta=None, out=None):
    """As smoothquant_fold_fp8 with one weight step max |W-hat| / 448 for the whole tensor (codes saturated)."""
    return _fold("smoothquant_fold_fp8_per_tensor", act_absmax, w, alpha, eps, norm, gamma, beta, out)


def _fold(fn, act_absmax, w, alpha, eps, norm, gamma, beta, out):
    _dev(w, "w", _ACT)
    n, k = w.shape
    _dev(act_absmax, "act_absmax", torch.float32, (k,))
    _dev(gamma, "gamma", torch.float32, (k,))
    _dev(beta, "beta", torch.float32, (k,))
    out = dict(out or {})
    dev = w.device
    out.setdefault("s", torch.empty(k, dtype=torch.float32, device=dev))
    out.setdefault("gamma_f", torch.empty(k, dtype=torch.float32, device=dev))
    if beta is not None:
        out.setdefault("beta_f", torch.empty(k, dtype=torch.float32, device=dev))
    else:
        out["beta_f"] = None
    code_dt = torch.uint8 if "_fp8" in fn else torch.int8
    out.setdefault("wq", torch.empty(n, k, dtype=code_dt, device=dev))
    out.setdefault("w_scale", torch.empty(n, dtype=torch.float32, device=dev))
    for key, shp, dt in [("s", (k,), torch.float32), ("gamma_f", (k,), torch.float32),
                         ("beta_f", (k,), torch.float32), ("wq", (n, k), code_dt), ("w_scale", (n,), torch.float32)]:
        _dev(out[key], key, dt, shp)
    with torch.cuda.device(dev):
        _check(fn, getattr(lib, fn)(
            _ptr(act_absmax), _ptr(w), _DT[w.dtype], n, k, float(alpha), eps, _NORM[norm], _ptr(gamma), _ptr(beta),
            _ptr(out["s"]), _ptr(out["gamma_f"]), _ptr(out["beta_f"]), _ptr(out["wq"]), _ptr(out["w_scale"]),
            _stream(w)))
    return out


def sq_norm_quant(x, norm="none", gamma_f=None, beta_f=None, eps=1e-5, xq=None, x_scale=None):
    """Fused norm (folded gamma', beta') + per-token INT8: returns (xq [M, K] int8, x_scale [M] fp32)."""
    return _nq("sq_norm_quant", x, norm, gamma_f, beta_f, eps, xq, x_scale)


def sq_norm_quant_fp8(x, norm="none", gamma_f=None, beta_f=None, eps=1e-5, xq=None, x_scale=None):
    """Fused norm + per-token FP8 (OCP E4M3): returns (xq [M, K] uint8 codes, x_scale [M] fp32 = absmax / 448)."""
    return _nq("sq_norm_quant_fp8", x, norm, gamma_f, beta_f, eps, xq, x_scale)


def sq_norm_quant_per_tensor(x, norm="none", gamma_f=None, beta_f=None, eps=1e-5, xq=None, x_scale=None):
    """Fused norm + INT8 with one dynamic step for the whole tensor (x_scale holds it repeated)."""
    return _nq("sq_norm_quant_per_tensor", x, norm, gamma_f, beta_f, eps, xq, x_scale)


def sq_norm_quant_static(x, step, norm="none", gamma_f=None, beta_f=None, eps=1e-5, xq=None, x_scale=None):
    """Fused norm + INT8 with a static step (a [1] fp32 device tensor), codes clipped to +-127."""
    _dev(step, "step", torch.float32, (1,))
    return _nq("sq_norm_quant_static", x, norm, gamma_f, beta_f, eps, xq, x_scale, step)


def sq_norm_quant_fp8_per_tensor(x, norm="none", gamma_f=None, beta_f=None, eps=1e-5, xq=None, x_scale=None):
    """Fused norm + FP8 (E4M3) codes with one dynamic step max |y| / 448 for the whole tensor."""
    return _nq("sq_norm_quant_fp8_per_tensor", x, norm, gamma_f, beta_f, eps, xq, x_scale)


def sq_norm_quant_fp8_static(x, step, norm="none", gamma_f=None, beta_f=None, eps=1e-5, xq=None, x_scale=None):
    """Fused norm + FP8 (E4M3) codes with a static step (a [1] fp32 device tensor), saturated to +-448."""
    _dev(step, "step", torch.float32, (1,))
    return _nq("sq_norm_quant_fp8_static", x, norm, gamma_f, beta_f, eps, xq, x_scale, step)


def sq_static_step_fp8(act_absmax, s, step=None):
    """Static FP8 activation step fl32(max_j fl32(a_j / s_j) / 448) into a [1] fp32 tensor."""
    return _static_step("sq_static_step_fp8", act_absmax, s, step)


def sq_static_step(act_absmax, s, step=None):
    """Static activation step fl32(max_j fl32(a_j / s_j) / 127) into a [1] fp32 tensor."""
    return _static_step("sq_static_step", act_absmax, s, step)


def _static_step(fn, act_absmax, s, step):
    k = act_absmax.shape[0]
    _dev(act_absmax, "act_absmax", torch.float32, (k,))
    _dev(s, "s", torch.float32, (k,))
    if step is None:
        step = torch.empty(1, dtype=torch.float32, device=s.device)
    _dev(step, "step", torch.float32, (1,))
    with torch.cuda.device(s.device):
        _check(fn, getattr(lib, fn)(_ptr(act_absmax), _ptr(s), k, _ptr(step), _stream(s)))
    return step


def _nq(fn, x, norm, gamma_f, beta_f, eps, xq, x_scale, *step):
    _dev(x, "x", _ACT)
    m, k = x.shape
    _dev(gamma_f, "gamma_f", torch.float32, (k,))
    _dev(beta_f, "beta_f", torch.float32, (k,))
    code_dt = torch.uint8 if "_fp8" in fn else torch.int8
    if xq is None:
        xq = torch.empty(m, k, dtype=code_dt, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _dev(xq, "xq", code_dt, (m, k))
    _dev(x_scale, "x_scale", torch.float32, (m,))
    with torch.cuda.device(x.device):
        _check(fn, getattr(lib, fn)(
            _ptr(x), _DT[x.dtype], m, k, _NORM[norm], _ptr(gamma_f), _ptr(beta_f), eps, *[_ptr(t) for t in step],
            _ptr(xq), _ptr(x_scale), _stream(x)))
    return xq, x_scale


def sq_w8a8_gemm(xq, x_scale, wq, w_scale, bias=None, out_dtype=torch.float16, y=None):
    """y [M, N] = dequant(xq @ wq^T); out_dtype torch.int32 returns the raw accumulator."""
    _dev(xq, "xq", torch.int8)
    _dev(wq, "wq", torch.int8)
    m, k = xq.shape
    n = wq.shape[0]
    if wq.shape[1] != k:
        raise ValueError(f"K mismatch: xq {tuple(xq.shape)} vs wq {tuple(wq.shape)}")
    if out_dtype != torch.int32:
        _dev(x_scale, "x_scale", torch.float32, (m,))
        _dev(w_scale, "w_scale", torch.float32, (n,))
        _dev(bias, "bias", torch.float32, (n,))
    if y is None:
        y = torch.empty(m, n, dtype=out_dtype, device=xq.device)
    _dev(y, "y", out_dtype, (m, n))
    with torch.cuda.device(xq.device):
        _check("sq_w8a8_gemm", lib.sq_w8a8_gemm(
            _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y), _DT[y.dtype], m, n, k,
            _stream(xq)))
    return y


def sq_fp8_gemm(xq, x_scale, wq, w_scale, bias=None, out_dtype=torch.float16, y=None):
    """y [M, N] = dequant(E4M3(xq) @ E4M3(wq)^T), binary32 accumulation; xq, wq uint8 E4M3 codes."""
    _dev(xq, "xq", torch.uint8)
    _dev(wq, "wq", torch.uint8)
    m, k = xq.shape
    n = wq.shape[0]
    if wq.shape[1] != k:
        raise ValueError(f"K mismatch: xq {tuple(xq.shape)} vs wq {tuple(wq.shape)}")
    _dev(x_scale, "x_scale", torch.float32, (m,))
    _dev(w_scale, "w_scale", torch.float32, (n,))
    _dev(bias, "bias", torch.float32, (n,))
    if y is None:
        y = torch.empty(m, n, dtype=out_dtype, device=xq.device)
    _dev(y, "y", out_dtype, (m, n))
    with torch.cuda.device(xq.device):
        _check("sq_fp8_gemm", lib.sq_fp8_gemm(
            _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y), _DT[y.dtype], m, n, k,
            _stream(xq)))
    return y


def sq_llm_int8_workspace(m, n, k):
    """Workspace layout of sq_llm_int8_linear for M x N x K: a dict of byte offsets and the total."""
    lay = _LlmLayout()
    _check("sq_llm_int8_workspace", lib.sq_llm_int8_workspace(int(m), int(n), int(k), ctypes.byref(lay)))
    return {name: int(getattr(lay, name)) for name in LLM_INT8_FIELDS}


def sq_llm_int8_linear(x, w, wq, w_scale, norm="none", gamma=None, beta=None, eps=1e-5, tau=6.0, bias=None,
                       out_dtype=torch.float16, y=None, workspace=None):
    """LLM.int8() decomposition: y [M, N] = 16-bit product of the channels whose |y| reaches tau + the
    dequantised INT8 product of the rest. x [M, K], w [N, K] (the 16-bit weights), wq [N, K] int8 and
    w_scale [N] (per-output-channel INT8 of w). Returns (y, workspace); the workspace (uint8, allocated
    here when None) holds the parts listed by sq_llm_int8_workspace."""
    _dev(x, "x", _ACT)
    _dev(w, "w", _ACT)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs w {tuple(w.shape)}")
    _dev(wq, "wq", torch.int8, (n, k))
    _dev(w_scale, "w_scale", torch.float32, (n,))
    _dev(gamma, "gamma", torch.float32, (k,))
    _dev(beta, "beta", torch.float32, (k,))
    _dev(bias, "bias", torch.float32, (n,))
    need = sq_llm_int8_workspace(m, n, k)["total"]
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    if y is None:
        y = torch.empty(m, n, dtype=out_dtype, device=x.device)
    _dev(y, "y", out_dtype, (m, n))
    with torch.cuda.device(x.device):
        _check("sq_llm_int8_linear", lib.sq_llm_int8_linear(
            _ptr(x), _DT[x.dtype], m, k, _NORM[norm], _ptr(gamma), _ptr(beta), eps, float(tau), _ptr(w), _DT[w.dtype],
            _ptr(wq), _ptr(w_scale), n, _ptr(bias), _ptr(y), _DT[y.dtype], _ptr(workspace), workspace.numel(),
            _stream(x)))
    return y, workspace


def llm_int8_parts(workspace, m, n, k, w_dtype=torch.float16):
    """Views of the parts an sq_llm_int8_linear call left in its workspace (after synchronisation):
    count, idx, absmax, gamma_m, beta_m, stats [M, 2], xq [M, K], x_scale [M], x16 [M, P] and w16 [N, P]
    (16-bit values, P = |O| padded to 32), deq [M, N]."""
    lay = sq_llm_int8_workspace(m, n, k)
    half = torch.bfloat16 if w_dtype == torch.bfloat16 else torch.float16

    def view(name, dtype, count):
        nbytes = count * torch.empty(0, dtype=dtype).element_size()
        return workspace[lay[name]:lay[name] + nbytes].view(dtype)
    count = int(view("count", torch.int32, 1).item())
    p = (count + 31) // 32 * 32
    return {"count": count, "idx": view("idx", torch.int32, k)[:count],
            "absmax": view("absmax", torch.float32, k), "gamma_m": view("gamma_m", torch.float32, k),
            "beta_m": view("beta_m", torch.float32, k), "stats": view("stats", torch.float32, 2 * m).view(m, 2),
            "xq": view("xq", torch.int8, m * k).view(m, k), "x_scale": view("x_scale", torch.float32, m),
            "x16": view("x16", half, m * p).view(m, p), "w16": view("w16", half, n * p).view(n, p),
            "deq": view("deq", torch.float32, m * n).view(m, n)}


def sq_llm_int8_linear_noalloc(x, w, wq, w_scale, norm="none", gamma=None, beta=None, eps=1e-5, tau=6.0, bias=None,
                               out_dtype=torch.float16, y=None):
    """sq_llm_int8_linear with the library's fixed device scratch as its workspace (no allocation in the
    call; y is allocated here only when None). Shapes whose workspace exceeds SQ_NOALLOC_SCRATCH_BYTES
    raise SmoothQuantError (SQ_ERR_TOO_LARGE)."""
    _dev(x, "x", _ACT)
    _dev(w, "w", _ACT)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs w {tuple(w.shape)}")
    _dev(wq, "wq", torch.int8, (n, k))
    _dev(w_scale, "w_scale", torch.float32, (n,))
    _dev(gamma, "gamma", torch.float32, (k,))
    _dev(beta, "beta", torch.float32, (k,))
    _dev(bias, "bias", torch.float32, (n,))
    if y is None:
        y = torch.empty(m, n, dtype=out_dtype, device=x.device)
    _dev(y, "y", out_dtype, (m, n))
    with torch.cuda.device(x.device):
        _check("sq_llm_int8_linear_noalloc", lib.sq_llm_int8_linear_noalloc(
            _ptr(x), _DT[x.dtype], m, k, _NORM[norm], _ptr(gamma), _ptr(beta), eps, float(tau), _ptr(w), _DT[w.dtype],
            _ptr(wq), _ptr(w_scale), n, _ptr(bias), _ptr(y), _DT[y.dtype], _stream(x)))
    return y
