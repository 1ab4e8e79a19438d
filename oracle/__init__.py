"""CPU double-precision oracle for the row-wise LayerNorm / RMSNorm forward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this package; the product package
(`rmsnorm_forward_amd`) never does.  The arithmetic lives in `oracle.c`
(plain C, IEEE double, left-to-right loops); this module only builds and
loads it and marshals numpy arrays.

Storage conventions (shared with the input generators in `workloads`):
  "f32"  -> numpy float32 array
  "f16"  -> numpy float16 array (IEEE binary16)
  "bf16" -> numpy uint16 array holding bfloat16 bit patterns
  "f64"  -> numpy float64 array (oracle-only; the decimal example rows)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "f64": np.float64}

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fno-unsafe-math-optimizations", "-shared", "-fPIC"]


def compile_c(src: str, out: str) -> str:
    """Compile an oracle source file into a shared library at `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        compile_c(SRC, LIB)
    return LIB


def eps_as_kernel_sees(eps: float) -> float:
    """The ABI passes eps as a C float; the oracle uses that exact value."""
    return float(np.float32(eps))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check_storage(a, dtype, n=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    want = NP_STORAGE[dtype]
    if a.dtype != want:
        raise TypeError(f"oracle: expected {np.dtype(want)} storage for {dtype}, got {a.dtype}")
    if n is not None and a.size != n:
        raise ValueError(f"oracle: expected {n} elements, got {a.size}")
    return a


class Oracle:
    """ctypes front end of one build of oracle.c."""

    def __init__(self, libpath: str):
        lib = ctypes.CDLL(libpath)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.oracle_ln_fwd.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64,
                                      ctypes.c_double, vp, vp, vp]
        lib.oracle_ln_fwd.restype = ctypes.c_int
        lib.oracle_rms_fwd.argtypes = [vp, vp, ctypes.c_int, i64, i64,
                                       ctypes.c_double, vp, vp]
        lib.oracle_rms_fwd.restype = ctypes.c_int
        lib.oracle_add_rms_fwd.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64,
                                           ctypes.c_double, vp, vp, vp]
        lib.oracle_add_rms_fwd.restype = ctypes.c_int
        lib.oracle_ln_bwd.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_ln_bwd.restype = ctypes.c_int
        lib.oracle_rms_bwd.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, vp, vp, vp]
        lib.oracle_rms_bwd.restype = ctypes.c_int
        lib.oracle_quant_e4m3.argtypes = [vp, i64, ctypes.c_double, vp]
        lib.oracle_quant_e4m3.restype = None
        lib.oracle_round.argtypes = [vp, i64, ctypes.c_int, vp]
        lib.oracle_round.restype = None
        lib.oracle_widen.argtypes = [vp, i64, ctypes.c_int, vp]
        lib.oracle_widen.restype = None
        self.lib = lib

    def ln_fwd(self, x, gamma, beta, dtype: str, eps: float, exact_eps: bool = False):
        """LayerNorm forward of x[M, N] in double -> (y, mean, rstd) float64.

        eps is rounded to float32 first (what the ABI receives) unless
        exact_eps is set (used only by the closed-form pins)."""
        x = _check_storage(x, dtype)
        M, N = x.shape
        gamma = _check_storage(gamma, dtype, N)
        beta = _check_storage(beta, dtype, N)
        y = np.empty((M, N), np.float64)
        mean = np.empty(M, np.float64)
        rstd = np.empty(M, np.float64)
        e = float(eps) if exact_eps else eps_as_kernel_sees(eps)
        rc = self.lib.oracle_ln_fwd(_ptr(x), _ptr(gamma), _ptr(beta), DTYPE_CODE[dtype],
                                    M, N, e, _ptr(y), _ptr(mean), _ptr(rstd))
        if rc != 0:
            raise ValueError("oracle_ln_fwd rejected its arguments")
        return y, mean, rstd

    def rms_fwd(self, x, gamma, dtype: str, eps: float, exact_eps: bool = False):
        """RMSNorm forward of x[M, N] in double -> (y, rstd) float64."""
        x = _check_storage(x, dtype)
        M, N = x.shape
        gamma = _check_storage(gamma, dtype, N)
        y = np.empty((M, N), np.float64)
        rstd = np.empty(M, np.float64)
        e = float(eps) if exact_eps else eps_as_kernel_sees(eps)
        rc = self.lib.oracle_rms_fwd(_ptr(x), _ptr(gamma), DTYPE_CODE[dtype], M, N,
                                     e, _ptr(y), _ptr(rstd))
        if rc != 0:
            raise ValueError("oracle_rms_fwd rejected its arguments")
        return y, rstd

    def add_rms_fwd(self, x, res, gamma, dtype: str, eps: float, exact_eps: bool = False):
        """Residual add then RMSNorm of x[M, N] + res[M, N] -> (h, y, rstd):
        h the rounded sum in storage `dtype`, y and rstd float64."""
        x = _check_storage(x, dtype)
        M, N = x.shape
        res = _check_storage(res, dtype, M * N)
        gamma = _check_storage(gamma, dtype, N)
        h = np.empty((M, N), NP_STORAGE[dtype])
        y = np.empty((M, N), np.float64)
        rstd = np.empty(M, np.float64)
        e = float(eps) if exact_eps else eps_as_kernel_sees(eps)
        rc = self.lib.oracle_add_rms_fwd(_ptr(x), _ptr(res), _ptr(gamma), DTYPE_CODE[dtype], M, N,
                                         e, _ptr(h), _ptr(y), _ptr(rstd))
        if rc != 0:
            raise ValueError("oracle_add_rms_fwd rejected its arguments")
        return h, y, rstd

    def ln_bwd(self, dy, x, gamma, dtype: str, mean, rstd):
        """LayerNorm backward from the forward's mean / rstd (any float
        arrays, used as doubles) -> (dx, dgamma, dbeta) float64."""
        x = _check_storage(x, dtype)
        M, N = x.shape
        dy = _check_storage(dy, dtype, M * N)
        gamma = _check_storage(gamma, dtype, N)
        mean = np.ascontiguousarray(mean, np.float64)
        rstd = np.ascontiguousarray(rstd, np.float64)
        dx = np.empty((M, N), np.float64)
        dg = np.empty(N, np.float64)
        db = np.empty(N, np.float64)
        rc = self.lib.oracle_ln_bwd(_ptr(dy), _ptr(x), _ptr(gamma), DTYPE_CODE[dtype], M, N, _ptr(mean),
                                    _ptr(rstd), _ptr(dx), _ptr(dg), _ptr(db))
        if rc != 0:
            raise ValueError("oracle_ln_bwd rejected its arguments")
        return dx, dg, db

    def rms_bwd(self, dy, x, gamma, dtype: str, rstd):
        """RMSNorm backward from the forward's rstd -> (dx, dgamma) float64."""
        x = _check_storage(x, dtype)
        M, N = x.shape
        dy = _check_storage(dy, dtype, M * N)
        gamma = _check_storage(gamma, dtype, N)
        rstd = np.ascontiguousarray(rstd, np.float64)
        dx = np.empty((M, N), np.float64)
        dg = np.empty(N, np.float64)
        rc = self.lib.oracle_rms_bwd(_ptr(dy), _ptr(x), _ptr(gamma), DTYPE_CODE[dtype], M, N, _ptr(rstd),
                                     _ptr(dx), _ptr(dg))
        if rc != 0:
            raise ValueError("oracle_rms_bwd rejected its arguments")
        return dx, dg

    def quant_e4m3(self, v, scale: float):
        """OCP E4M3 codes (uint8) of v / scale, saturated to +-448, RNE."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, np.uint8)
        self.lib.oracle_quant_e4m3(_ptr(v), v.size, float(np.float32(scale)), _ptr(out))
        return out

    def rms_fp8_fwd(self, x, gamma, dtype: str, eps: float, scale: float):
        """RMSNorm with FP8 output -> (codes uint8, y float64 before
        quantisation, rstd)."""
        y, rstd = self.rms_fwd(x, gamma, dtype, eps)
        return self.quant_e4m3(y, scale), y, rstd

    def add_rms_fp8_fwd(self, x, res, gamma, dtype: str, eps: float, scale: float):
        """Residual add + RMSNorm with FP8 output -> (h, codes, y, rstd)."""
        h, y, rstd = self.add_rms_fwd(x, res, gamma, dtype, eps)
        return h, self.quant_e4m3(y, scale), y, rstd

    def round_to(self, v, dtype: str):
        """Round float64 values to storage `dtype`, direct round-to-nearest-even."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, NP_STORAGE[dtype])
        self.lib.oracle_round(_ptr(v), v.size, DTYPE_CODE[dtype], _ptr(out))
        return out

    def widen(self, a, dtype: str):
        """Exact float64 value of stored elements."""
        a = _check_storage(a, dtype)
        out = np.empty(a.shape, np.float64)
        self.lib.oracle_widen(_ptr(a), a.size, DTYPE_CODE[dtype], _ptr(out))
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build(force=False)
        _default = Oracle(LIB)
    return _default


def ln_fwd(x, gamma, beta, dtype: str, eps: float):
    return default().ln_fwd(x, gamma, beta, dtype, eps)


def rms_fwd(x, gamma, dtype: str, eps: float):
    return default().rms_fwd(x, gamma, dtype, eps)


def add_rms_fwd(x, res, gamma, dtype: str, eps: float):
    return default().add_rms_fwd(x, res, gamma, dtype, eps)


def ln_bwd(dy, x, gamma, dtype: str, mean, rstd):
    return default().ln_bwd(dy, x, gamma, dtype, mean, rstd)


def rms_bwd(dy, x, gamma, dtype: str, rstd):
    return default().rms_bwd(dy, x, gamma, dtype, rstd)


def quant_e4m3(v, scale: float):
    return default().quant_e4m3(v, scale)


def rms_fp8_fwd(x, gamma, dtype: str, eps: float, scale: float):
    return default().rms_fp8_fwd(x, gamma, dtype, eps, scale)


def add_rms_fp8_fwd(x, res, gamma, dtype: str, eps: float, scale: float):
    return default().add_rms_fp8_fwd(x, res, gamma, dtype, eps, scale)


def round_to(v, dtype: str):
    return default().round_to(v, dtype)


def widen(a, dtype: str):
    return default().widen(a, dtype)
