"""rmsnorm_forward_amd -- row-wise LayerNorm / RMSNorm forward on AMD MI355X.

A thin binding of libmi355norm.so (C ABI in include/mi355norm.h): ctypes,
with the per-call entry points through a small CPython module when built.
Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments.  PyTorch is used for device memory and streams.

Two layers:
  * ln_fwd / rms_fwd / add_rms_fwd / rms_fp8_fwd / add_rms_fp8_fwd /
    norm_fwd (row strides) / norm_fwd_noalloc (the same, allocating
    nothing) / ln_bwd / rms_bwd / norm_bwd (row strides) /
    norm_status_str /
    norm_last_error / norm_describe / norm_bwd_describe -- the C ABI entry
    points under the same names, taking raw device addresses (ints) and
    returning the status code;
  * layer_norm / rms_norm / fused_add_rms_norm / rms_norm_fp8 /
    fused_add_rms_norm_fp8 -- the same calls on torch tensors: they allocate
    y (and fp32 mean / rstd), pass the current stream, and raise
    RuntimeError with the library's message on a non-zero status;
    layer_norm_backward / rms_norm_backward take the saved statistics, and
    layer_norm_autograd / rms_norm_autograd wrap forward and backward as
    torch autograd functions.

Importing this package raises ImportError if the library has not been built
(`python rmsnorm_forward_amd/build.py`): there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi355norm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python rmsnorm_forward_amd/build.py` "
        "(hipcc, gfx950).  There is no non-HIP fallback.")

# The library is handed torch's allocations and stream handles, so it must
# run on the HIP runtime torch runs on.  torch ships its own libamdhip64 with
# the same soname as the system one; loading torch first makes the dynamic
# loader bind the library to that copy instead of mapping a second runtime.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # a process without torch uses the system runtime
    _torch = None

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _f32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
for _name in ("ln_fwd", "rms_fwd"):
    _fn = getattr(_lib, _name)
    _fn.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _vp]
    _fn.restype = _int
_lib.add_rms_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _vp]
_lib.add_rms_fwd.restype = _int
_lib.rms_fp8_fwd.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _int, _vp]
_lib.rms_fp8_fwd.restype = _int
_lib.add_rms_fp8_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _f32, _int, _vp]
_lib.add_rms_fp8_fwd.restype = _int
_lib.norm_status_str.argtypes = [_int]
_lib.norm_status_str.restype = ctypes.c_char_p
_lib.norm_last_error.argtypes = []
_lib.norm_last_error.restype = ctypes.c_char_p
_lib.norm_describe.argtypes = [_int, _i64, _i64, _int, _int, ctypes.c_char_p, _int]
_lib.norm_describe.restype = _int
_lib.ln_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _vp]
_lib.ln_bwd.restype = _int
_lib.rms_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _vp]
_lib.rms_bwd.restype = _int
_lib.norm_bwd_describe.argtypes = [_int, _i64, _i64, _int, _int, ctypes.c_char_p, _int]
_lib.norm_bwd_describe.restype = _int

NORM_F32, NORM_F16, NORM_BF16 = 0, 1, 2
NORM_OK = 0
NORM_ERR_NULL_ARG, NORM_ERR_BAD_SHAPE, NORM_ERR_BAD_DTYPE, NORM_ERR_BAD_EPS = 1, 2, 3, 4
NORM_ERR_BAD_ARG, NORM_ERR_ALIAS, NORM_ERR_HIP, NORM_ERR_SCRATCH = 5, 6, 7, 8
STATUS = {0: "NORM_OK", 1: "NORM_ERR_NULL_ARG", 2: "NORM_ERR_BAD_SHAPE", 3: "NORM_ERR_BAD_DTYPE",
          4: "NORM_ERR_BAD_EPS", 5: "NORM_ERR_BAD_ARG", 6: "NORM_ERR_ALIAS", 7: "NORM_ERR_HIP",
          8: "NORM_ERR_SCRATCH"}
DTYPE_NAMES = {"f32": NORM_F32, "f16": NORM_F16, "bf16": NORM_BF16}


def _addr(p):
    return None if not p else int(p)


# ---------------------------------------------------------------------------
# C ABI, same names
# ---------------------------------------------------------------------------

def ln_fwd(x, gamma, beta, y, mean, rstd, M, N, eps, dtype, stream) -> int:
    """LayerNorm forward on device addresses; returns the norm_status code."""
    return _lib.ln_fwd(_addr(x), _addr(gamma), _addr(beta), _addr(y), _addr(mean), _addr(rstd),
                       int(M), int(N), float(eps), int(dtype), _addr(stream))


def rms_fwd(x, gamma, beta, y, mean, rstd, M, N, eps, dtype, stream) -> int:
    """RMSNorm forward on device addresses; returns the norm_status code."""
    return _lib.rms_fwd(_addr(x), _addr(gamma), _addr(beta), _addr(y), _addr(mean), _addr(rstd),
                        int(M), int(N), float(eps), int(dtype), _addr(stream))


def add_rms_fwd(x, residual, gamma, y, residual_out, rstd, M, N, eps, dtype, stream) -> int:
    """Residual add then RMSNorm on device addresses; returns the norm_status code."""
    return _lib.add_rms_fwd(_addr(x), _addr(residual), _addr(gamma), _addr(y), _addr(residual_out),
                            _addr(rstd), int(M), int(N), float(eps), int(dtype), _addr(stream))


def rms_fp8_fwd(x, gamma, y, rstd, M, N, eps, scale, dtype, stream) -> int:
    """RMSNorm with FP8 (E4M3) output on device addresses; returns the status."""
    return _lib.rms_fp8_fwd(_addr(x), _addr(gamma), _addr(y), _addr(rstd), int(M), int(N), float(eps),
                            float(scale), int(dtype), _addr(stream))


def add_rms_fp8_fwd(x, residual, gamma, y, residual_out, rstd, M, N, eps, scale, dtype, stream) -> int:
    """Residual add + RMSNorm with FP8 (E4M3) output on device addresses."""
    return _lib.add_rms_fp8_fwd(_addr(x), _addr(residual), _addr(gamma), _addr(y), _addr(residual_out),
                                _addr(rstd), int(M), int(N), float(eps), float(scale), int(dtype),
                                _addr(stream))


def ln_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, M, N, dtype, stream) -> int:
    """LayerNorm backward on device addresses (dgamma / dbeta fp32 [N] or
    None); returns the norm_status code."""
    return _lib.ln_bwd(_addr(dy), _addr(x), _addr(gamma), _addr(mean), _addr(rstd), _addr(dx), _addr(dgamma),
                       _addr(dbeta), int(M), int(N), int(dtype), _addr(stream))


def rms_bwd(dy, x, gamma, rstd, dx, dgamma, M, N, dtype, stream) -> int:
    """RMSNorm backward on device addresses; returns the norm_status code."""
    return _lib.rms_bwd(_addr(dy), _addr(x), _addr(gamma), _addr(rstd), _addr(dx), _addr(dgamma), int(M),
                        int(N), int(dtype), _addr(stream))


# The per-call entry points above go through the CPython module built from
# csrc/pycalls.c when it is present: the same library calls with the same
# arguments and results, about 1.7 us cheaper per call than ctypes'
# conversion of their arguments.  It is handed the addresses of the loaded
# library's entry points, so both paths call one copy of the library.
try:
    from . import _calls
except ImportError:  # not built: the ctypes calls above stay
    _calls = None
if _calls is not None:
    _calls._bind(*(ctypes.cast(getattr(_lib, _n), ctypes.c_void_p).value
                   for _n in ("ln_fwd", "rms_fwd", "add_rms_fwd", "rms_fp8_fwd", "add_rms_fp8_fwd", "ln_bwd",
                              "rms_bwd")))
    ln_fwd, rms_fwd, add_rms_fwd = _calls.ln_fwd, _calls.rms_fwd, _calls.add_rms_fwd
    rms_fp8_fwd, add_rms_fp8_fwd = _calls.rms_fp8_fwd, _calls.add_rms_fp8_fwd
    ln_bwd, rms_bwd = _calls.ln_bwd, _calls.rms_bwd


class NormArgs(ctypes.Structure):
    """norm_args of include/mi355norm.h."""
    _fields_ = [("op", _int), ("dtype", _int), ("M", _i64), ("N", _i64),
                ("x", _vp), ("ld_x", _i64), ("residual", _vp), ("ld_residual", _i64),
                ("gamma", _vp), ("beta", _vp), ("y", _vp), ("ld_y", _i64),
                ("residual_out", _vp), ("ld_residual_out", _i64), ("mean", _vp), ("rstd", _vp),
                ("eps", _f32), ("scale", _f32)]


_lib.norm_fwd.argtypes = [ctypes.POINTER(NormArgs), _vp]
_lib.norm_fwd.restype = _int
OPS = {"ln": 0, "rms": 1, "add_rms": 2, "rms_fp8": 3, "add_rms_fp8": 4}


def norm_fwd(op, dtype, M, N, x, y, *, ld_x=0, residual=None, ld_residual=0, gamma=None, beta=None,
             ld_y=0, residual_out=None, ld_residual_out=0, mean=None, rstd=None, eps=1e-5, scale=1.0,
             stream=None) -> int:
    """Any operation with row strides (elements; 0 = N), on device addresses;
    returns the norm_status code."""
    a = NormArgs(OPS.get(op, op), DTYPE_NAMES.get(dtype, dtype), int(M), int(N), _addr(x), int(ld_x),
                 _addr(residual), int(ld_residual), _addr(gamma), _addr(beta), _addr(y), int(ld_y),
                 _addr(residual_out), int(ld_residual_out), _addr(mean), _addr(rstd), float(eps), float(scale))
    return _lib.norm_fwd(ctypes.byref(a), _addr(stream))


_lib.norm_fwd_noalloc.argtypes = [ctypes.POINTER(NormArgs), _vp]
_lib.norm_fwd_noalloc.restype = _int


def norm_fwd_noalloc(op, dtype, M, N, x, y, *, ld_x=0, residual=None, ld_residual=0, gamma=None, beta=None,
                     ld_y=0, residual_out=None, ld_residual_out=0, mean=None, rstd=None, eps=1e-5, scale=1.0,
                     stream=None) -> int:
    """norm_fwd that allocates nothing (split rows use the library's fixed
    scratch); same arguments; returns the norm_status code."""
    a = NormArgs(OPS.get(op, op), DTYPE_NAMES.get(dtype, dtype), int(M), int(N), _addr(x), int(ld_x),
                 _addr(residual), int(ld_residual), _addr(gamma), _addr(beta), _addr(y), int(ld_y),
                 _addr(residual_out), int(ld_residual_out), _addr(mean), _addr(rstd), float(eps), float(scale))
    return _lib.norm_fwd_noalloc(ctypes.byref(a), _addr(stream))


class NormBwdArgs(ctypes.Structure):
    """norm_bwd_args of include/mi355norm.h."""
    _fields_ = [("op", _int), ("dtype", _int), ("M", _i64), ("N", _i64),
                ("dy", _vp), ("ld_dy", _i64), ("x", _vp), ("ld_x", _i64), ("gamma", _vp),
                ("mean", _vp), ("rstd", _vp), ("dx", _vp), ("ld_dx", _i64), ("dgamma", _vp), ("dbeta", _vp)]


_lib.norm_bwd.argtypes = [ctypes.POINTER(NormBwdArgs), _vp]
_lib.norm_bwd.restype = _int


def norm_bwd(op, dtype, M, N, dy, x, dx, *, ld_dy=0, ld_x=0, ld_dx=0, gamma=None, mean=None, rstd=None,
             dgamma=None, dbeta=None, stream=None) -> int:
    """ln_bwd (op "ln") or rms_bwd (op "rms") with row strides (elements;
    0 = N), on device addresses; returns the norm_status code."""
    a = NormBwdArgs(OPS.get(op, op), DTYPE_NAMES.get(dtype, dtype), int(M), int(N), _addr(dy), int(ld_dy),
                    _addr(x), int(ld_x), _addr(gamma), _addr(mean), _addr(rstd), _addr(dx), int(ld_dx),
                    _addr(dgamma), _addr(dbeta))
    return _lib.norm_bwd(ctypes.byref(a), _addr(stream))


def norm_status_str(status: int) -> str:
    return _lib.norm_status_str(int(status)).decode()


def norm_last_error() -> str:
    """The HIP failure behind this thread's last NORM_ERR_HIP ("" if none)."""
    return _lib.norm_last_error().decode()


def norm_describe(op: str, M: int, N: int, dtype, aligned=True) -> str:
    """How the library would run this call (path, tile, grid); launches nothing.
    aligned: True (every pointer 16-byte aligned), False, or "x" (x alone is
    not: the realigned row kernel)."""
    code = OPS[op]
    dt = DTYPE_NAMES.get(dtype, dtype)
    buf = ctypes.create_string_buffer(256)
    al = 2 if aligned == "x" else int(bool(aligned))
    st = _lib.norm_describe(code, int(M), int(N), int(dt), al, buf, 256)
    if st != NORM_OK:
        raise RuntimeError(norm_status_str(st))
    return buf.value.decode()


def norm_bwd_describe(op: str, M: int, N: int, dtype, aligned: bool = True) -> str:
    """How ln_bwd (op "ln") or rms_bwd (op "rms") would run; launches nothing."""
    if op not in ("ln", "rms"):
        raise ValueError("op must be 'ln' or 'rms'")
    dt = DTYPE_NAMES.get(dtype, dtype)
    buf = ctypes.create_string_buffer(256)
    st = _lib.norm_bwd_describe(int(op == "rms"), int(M), int(N), int(dt), int(bool(aligned)), buf, 256)
    if st != NORM_OK:
        raise RuntimeError(norm_status_str(st))
    return buf.value.decode()


# ---------------------------------------------------------------------------
# torch tensors
# ---------------------------------------------------------------------------

def _torch_dtype_code(t):
    import torch
    m = {torch.float32: NORM_F32, torch.float16: NORM_F16, torch.bfloat16: NORM_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return m[t.dtype]


def _param(p, N, x):
    if p is None:
        return None
    if p.dtype != x.dtype or p.device != x.device or p.numel() != N:
        raise ValueError("gamma/beta must have N elements and x's dtype and device")
    return p.contiguous()


def _rows(t, N):
    """(M, N) view of t and its row stride: rows may be strided (a slice of
    a wider matrix), elements within a row must be contiguous; anything else
    is copied to a contiguous matrix."""
    if t.dim() >= 1 and t.stride(-1) == 1:
        try:
            v = t.view(-1, N)
            return v, (v.stride(0) if v.shape[0] > 1 else N)
        except RuntimeError:
            pass
    v = t.reshape(-1, N).contiguous()
    return v, N


def _check(st):
    if st != NORM_OK:
        extra = f" [{norm_last_error()}]" if st == NORM_ERR_HIP else ""
        raise RuntimeError(f"{STATUS.get(st, st)}: {norm_status_str(st)}{extra}")


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _run(op, x2, ldx, y, ldy, *, res=None, ldr=0, hout=None, ldh=0, gamma=None, beta=None, mean=None,
         rstd=None, eps=1e-5, scale=1.0):
    import torch
    M, N = x2.shape
    with torch.cuda.device(x2.device):
        stream = torch.cuda.current_stream(x2.device).cuda_stream
        _check(norm_fwd(op, _torch_dtype_code(x2), M, N, _ptr(x2), _ptr(y), ld_x=ldx, residual=_ptr(res),
                        ld_residual=ldr, gamma=_ptr(gamma), beta=_ptr(beta), ld_y=ldy,
                        residual_out=_ptr(hout), ld_residual_out=ldh, mean=_ptr(mean), rstd=_ptr(rstd),
                        eps=eps, scale=scale, stream=stream))


def layer_norm(x, gamma=None, beta=None, eps: float = 1e-5, want_stats: bool = True):
    """LayerNorm over the last dimension.  Returns (y, mean, rstd); y is
    contiguous, mean and rstd are fp32 [M] (None when want_stats is False).
    Rows of x may be strided (no copy)."""
    import torch
    N = x.shape[-1]
    x2, ldx = _rows(x, N)
    M = x2.shape[0]
    y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    mean = torch.empty(M, device=x.device, dtype=torch.float32) if want_stats else None
    rstd = torch.empty(M, device=x.device, dtype=torch.float32) if want_stats else None
    _run("ln", x2, ldx, y, N, gamma=_param(gamma, N, x), beta=_param(beta, N, x), mean=mean, rstd=rstd,
         eps=eps)
    return y.view(x.shape), mean, rstd


def rms_norm(x, gamma=None, eps: float = 1e-6, want_rstd: bool = True):
    """RMSNorm over the last dimension.  Returns (y, rstd); rstd is fp32 [M]
    (None when want_rstd is False).  Rows of x may be strided (no copy)."""
    import torch
    N = x.shape[-1]
    x2, ldx = _rows(x, N)
    M = x2.shape[0]
    y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    rstd = torch.empty(M, device=x.device, dtype=torch.float32) if want_rstd else None
    _run("rms", x2, ldx, y, N, gamma=_param(gamma, N, x), rstd=rstd, eps=eps)
    return y.view(x.shape), rstd


def _add_operands(x, residual, inplace):
    if residual.shape != x.shape or residual.dtype != x.dtype or residual.device != x.device:
        raise ValueError("residual must have x's shape, dtype and device")
    N = x.shape[-1]
    x2, ldx = _rows(x, N)
    r2, ldr = _rows(residual, N)
    if inplace and (r2.data_ptr() != residual.data_ptr() or
                    (residual.dim() > 1 and r2.shape[0] > 1 and residual.view(-1, N).stride(0) != ldr)):
        raise ValueError("inplace=True needs a residual whose rows can be viewed without a copy")
    return x2, ldx, r2, ldr


def fused_add_rms_norm(x, residual, gamma=None, eps: float = 1e-6, inplace: bool = False,
                       want_rstd: bool = True):
    """h = x + residual (rounded to x's dtype), y = RMSNorm(h) over the last
    dimension.  Returns (y, h, rstd).  With inplace=True, y is written into
    x and h into residual (their rows may be strided), the way a transformer
    block updates its residual stream."""
    import torch
    N = x.shape[-1]
    x2, ldx, r2, ldr = _add_operands(x, residual, inplace)
    if inplace and x2.data_ptr() != x.data_ptr():
        raise ValueError("inplace=True needs an x whose rows can be viewed without a copy")
    M = x2.shape[0]
    if inplace:
        y, ldy, h, ldh = x2, ldx, r2, ldr
    else:
        y, ldy = torch.empty((M, N), dtype=x.dtype, device=x.device), N
        h, ldh = torch.empty((M, N), dtype=x.dtype, device=x.device), N
    rstd = torch.empty(M, device=x.device, dtype=torch.float32) if want_rstd else None
    _run("add_rms", x2, ldx, y, ldy, res=r2, ldr=ldr, hout=h, ldh=ldh, gamma=_param(gamma, N, x),
         rstd=rstd, eps=eps)
    if inplace:
        return x, residual, rstd
    return y.view(x.shape), h.view(x.shape), rstd


def rms_norm_fp8(x, gamma=None, scale: float = 1.0, eps: float = 1e-6, want_rstd: bool = True):
    """RMSNorm over the last dimension with FP8 E4M3 output of y / scale.
    Returns (codes, rstd); codes is a torch.float8_e4m3fn tensor of x's shape."""
    import torch
    N = x.shape[-1]
    x2, ldx = _rows(x, N)
    M = x2.shape[0]
    y = torch.empty((M, N), dtype=torch.uint8, device=x.device)
    rstd = torch.empty(M, device=x.device, dtype=torch.float32) if want_rstd else None
    _run("rms_fp8", x2, ldx, y, N, gamma=_param(gamma, N, x), rstd=rstd, eps=eps, scale=scale)
    return y.view(torch.float8_e4m3fn).view(x.shape), rstd


def fused_add_rms_norm_fp8(x, residual, gamma=None, scale: float = 1.0, eps: float = 1e-6,
                           inplace: bool = False, want_rstd: bool = True):
    """h = x + residual, then RMSNorm of h with FP8 E4M3 output of y / scale.
    Returns (codes, h, rstd); with inplace=True h is written into residual."""
    import torch
    N = x.shape[-1]
    x2, ldx, r2, ldr = _add_operands(x, residual, inplace)
    M = x2.shape[0]
    y = torch.empty((M, N), dtype=torch.uint8, device=x.device)
    if inplace:
        h, ldh = r2, ldr
    else:
        h, ldh = torch.empty((M, N), dtype=x.dtype, device=x.device), N
    rstd = torch.empty(M, device=x.device, dtype=torch.float32) if want_rstd else None
    _run("add_rms_fp8", x2, ldx, y, N, res=r2, ldr=ldr, hout=h, ldh=ldh, gamma=_param(gamma, N, x),
         rstd=rstd, eps=eps, scale=scale)
    codes = y.view(torch.float8_e4m3fn).view(x.shape)
    return codes, (residual if inplace else h.view(x.shape)), rstd


def _bwd_run(op, dy, x, gamma, mean, rstd, want_dgamma, want_dbeta):
    """One norm_bwd call on tensors: dy and x may have strided rows (no
    copy); dx is allocated contiguous."""
    import torch
    if dy.shape != x.shape or dy.dtype != x.dtype or dy.device != x.device:
        raise ValueError("dy must have x's shape, dtype and device")
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    stats = [s for s in (mean, rstd) if s is not None]
    for s in stats:
        if s.dtype != torch.float32 or s.numel() != M or s.device != x.device:
            raise ValueError("mean / rstd must be fp32 with one value per row, on x's device")
    dy2, lddy = _rows(dy, N)
    x2, ldx = _rows(x, N)
    mean = mean.contiguous() if mean is not None else None
    rstd = rstd.contiguous()
    dx = torch.empty((M, N), dtype=x.dtype, device=x.device)
    dgamma = torch.empty(N, dtype=torch.float32, device=x.device) if want_dgamma else None
    dbeta = torch.empty(N, dtype=torch.float32, device=x.device) if want_dbeta else None
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        _check(norm_bwd(op, _torch_dtype_code(x), M, N, _ptr(dy2), _ptr(x2), _ptr(dx), ld_dy=lddy, ld_x=ldx,
                        ld_dx=N, gamma=_ptr(_param(gamma, N, x)), mean=_ptr(mean), rstd=_ptr(rstd),
                        dgamma=_ptr(dgamma), dbeta=_ptr(dbeta), stream=stream))
    return dx.view(x.shape), dgamma, dbeta


def layer_norm_backward(dy, x, mean, rstd, gamma=None, want_dgamma: bool = True, want_dbeta: bool = True):
    """Gradients of layer_norm from its saved fp32 mean and rstd: returns
    (dx, dgamma, dbeta); dx has x's shape and dtype, dgamma and dbeta are
    fp32 [N] (None when not wanted).  Rows of dy and x may be strided."""
    if mean is None:
        raise ValueError("layer_norm_backward needs the forward's mean")
    return _bwd_run("ln", dy, x, gamma, mean, rstd, want_dgamma, want_dbeta)


def rms_norm_backward(dy, x, rstd, gamma=None, want_dgamma: bool = True):
    """Gradients of rms_norm from its saved fp32 rstd: returns (dx, dgamma);
    dgamma is fp32 [N] (None when not wanted).  Rows of dy and x may be
    strided."""
    dx, dgamma, _ = _bwd_run("rms", dy, x, gamma, None, rstd, want_dgamma, False)
    return dx, dgamma


def _autograd():
    import torch

    class LayerNormFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, gamma, beta, eps):
            y, mean, rstd = layer_norm(x, gamma, beta, eps)
            ctx.save_for_backward(x, gamma, mean, rstd)
            ctx.has_beta = beta is not None
            return y

        @staticmethod
        def backward(ctx, dy):
            x, gamma, mean, rstd = ctx.saved_tensors
            need_g = gamma is not None and ctx.needs_input_grad[1]
            need_b = ctx.has_beta and ctx.needs_input_grad[2]
            dx, dg, db = layer_norm_backward(dy, x, mean, rstd, gamma, need_g, need_b)
            return (dx, dg.to(gamma.dtype) if need_g else None,
                    db.to(x.dtype) if need_b else None, None)

    class RMSNormFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, gamma, eps):
            y, rstd = rms_norm(x, gamma, eps)
            ctx.save_for_backward(x, gamma, rstd)
            return y

        @staticmethod
        def backward(ctx, dy):
            x, gamma, rstd = ctx.saved_tensors
            need_g = gamma is not None and ctx.needs_input_grad[1]
            dx, dg = rms_norm_backward(dy, x, rstd, gamma, need_g)
            return dx, dg.to(gamma.dtype) if need_g else None, None

    return LayerNormFn, RMSNormFn


_FNS = None


def layer_norm_autograd(x, gamma=None, beta=None, eps: float = 1e-5):
    """layer_norm as a differentiable torch op (backward: ln_bwd)."""
    global _FNS
    _FNS = _FNS or _autograd()
    return _FNS[0].apply(x, gamma, beta, eps)


def rms_norm_autograd(x, gamma=None, eps: float = 1e-6):
    """rms_norm as a differentiable torch op (backward: rms_bwd)."""
    global _FNS
    _FNS = _FNS or _autograd()
    return _FNS[1].apply(x, gamma, eps)


__all__ = ["ln_fwd", "rms_fwd", "add_rms_fwd", "rms_fp8_fwd", "add_rms_fp8_fwd", "norm_fwd", "NormArgs",
           "norm_status_str", "norm_last_error", "norm_describe", "layer_norm", "rms_norm",
           "fused_add_rms_norm", "rms_norm_fp8", "fused_add_rms_norm_fp8",
           "ln_bwd", "rms_bwd", "norm_bwd", "NormBwdArgs", "norm_bwd_describe", "layer_norm_backward", "rms_norm_backward",
           "layer_norm_autograd", "rms_norm_autograd",
           "NORM_F32", "NORM_F16", "NORM_BF16", "NORM_OK", "STATUS", "LIB_PATH", "OPS"]
