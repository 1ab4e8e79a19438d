"""Seeded synthetic inputs for the LayerNorm / RMSNorm forward workloads.

This module holds no normalisation arithmetic: it only draws random numbers
and stores them in the I/O dtype.  Both the oracle side (tests, CPU baseline)
and the HIP side (tests, bench, smoke) take their inputs from here.

Storage conventions:
  "f32"  -> numpy float32
  "f16"  -> numpy float16 (numpy's float32 -> binary16 conversion)
  "bf16" -> numpy uint16 of bfloat16 bit patterns (torch's CPU float32 ->
            bfloat16 conversion, round-to-nearest-even)

Random draws (numpy PCG64 `default_rng(seed)`):
  U(a, b)      a + (b - a) * u with u = rng.random(float32) in [0, 1)
  N(mu, sigma) float32 Box-Muller on two uniform streams, sigma being the
               standard deviation (numpy's `scale` convention)
Draw order inside a workload is x, then gamma, then beta.

The workloads follow the five configurations the norm is measured on; the
shapes and value distributions are those of the pages' own examples:
  * LN fp32 128x1024 with N(0,1) rows: the shape of the ROCm LayerNorm
    README's usage example ("Simple LayerNorm", section 6), plus the
    10-value large-mean row of "CUDA 算子工程" ch. 7, section 7.3.
  * RMS fp32 (B,T,C) = (8,1024,4096) and (64,1024,2048) with x ~ U(-1,1),
    weight ~ U(0,1): the shapes and the init of "CUDA算子优化(2)：RMSNorm",
    sections 2-5.
  * LN bf16 16384x8192 with large-mean rows and outlier channels: the
    stability stress of "CUDA 算子工程" ch. 7, section 7.3 (large-mean rows,
    activation outliers of a hundredfold).
  * LN bf16 with a non-power-of-two N (5120) and a very long row (2^20): the
    padding and segmented-read cases of "T3 讲解" part ②.
Follow-on operations at the LN bf16 16384x8192 shape: residual add +
RMSNorm, RMSNorm with FP8 output, and the LayerNorm / RMSNorm backward
("CUDA 算子工程" ch. 7, sections 7.7 and 7.9), with the upstream gradient
dy ~ N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "CONFIGS", "generate", "gen_ln_normal", "gen_rms_uniform", "gen_bwd",
           "gen_ln_stress", "gen_ln_large_mean", "check_row_f32", "to_storage",
           "normal", "uniform", "ELEM_BYTES"]

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


# --------------------------------------------------------------------------
# primitive draws
# --------------------------------------------------------------------------

def uniform(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    u = rng.random(shape, dtype=np.float32)
    return (np.float32(lo) + np.float32(hi - lo) * u).astype(np.float32, copy=False)


def normal(rng: np.random.Generator, shape, loc: float, scale: float) -> np.ndarray:
    """float32 normal samples by Box-Muller (Box & Muller, 1958)."""
    n = int(np.prod(shape))
    half = (n + 1) // 2
    u1 = rng.random(half, dtype=np.float32)
    u2 = rng.random(half, dtype=np.float32)
    rad = np.sqrt(np.float32(-2.0) * np.log1p(-u1))   # 1 - u1 in (0, 1]
    th = np.float32(2.0 * np.pi) * u2
    z = np.empty(2 * half, np.float32)
    z[0::2] = rad * np.cos(th)
    z[1::2] = rad * np.sin(th)
    z = z[:n].reshape(shape)
    if scale != 1.0:
        z *= np.float32(scale)
    if loc != 0.0:
        z += np.float32(loc)
    return z


def to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 values in the I/O dtype (see module docstring)."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return a32
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(a32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# workload families
# --------------------------------------------------------------------------

def gen_ln_normal(seed: int, M: int, N: int, dtype: str, loc: float = 0.0,
                  scale: float = 1.0, rng: np.random.Generator | None = None):
    """x ~ N(loc, scale), gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    x = normal(rng, (M, N), loc, scale)
    gamma = uniform(rng, (N,), 0.5, 1.5)
    beta = normal(rng, (N,), 0.0, 0.1)
    return {"x": to_storage(x, dtype), "gamma": to_storage(gamma, dtype),
            "beta": to_storage(beta, dtype)}


def gen_rms_uniform(seed: int, M: int, N: int, dtype: str):
    """x ~ U(-1, 1), weight ~ U(0, 1); RMSNorm has no beta."""
    rng = np.random.default_rng(seed)
    x = uniform(rng, (M, N), -1.0, 1.0)
    w = uniform(rng, (N,), 0.0, 1.0)
    return {"x": to_storage(x, dtype), "gamma": to_storage(w, dtype), "beta": None}


def gen_add_rms(seed: int, M: int, N: int, dtype: str):
    """Residual add + RMSNorm inputs: x ~ U(-1, 1) (a sublayer's output),
    residual ~ N(0, 1) (the residual stream), weight ~ U(0, 1)."""
    rng = np.random.default_rng(seed)
    x = uniform(rng, (M, N), -1.0, 1.0)
    res = normal(rng, (M, N), 0.0, 1.0)
    w = uniform(rng, (N,), 0.0, 1.0)
    return {"x": to_storage(x, dtype), "res": to_storage(res, dtype), "gamma": to_storage(w, dtype),
            "beta": None}


def gen_bwd(seed: int, M: int, N: int, dtype: str, op: str):
    """Backward inputs: the forward's inputs (LayerNorm: x ~ N(0, 1),
    gamma ~ U(0.5, 1.5); RMSNorm: x ~ U(-1, 1), weight ~ U(0, 1)), then the
    upstream gradient dy ~ N(0, 1).  The forward's mean / rstd are not drawn
    here: they are the forward pass's outputs."""
    rng = np.random.default_rng(seed)
    if op == "ln_bwd":
        x = normal(rng, (M, N), 0.0, 1.0)
        gamma = uniform(rng, (N,), 0.5, 1.5)
    elif op == "rms_bwd":
        x = uniform(rng, (M, N), -1.0, 1.0)
        gamma = uniform(rng, (N,), 0.0, 1.0)
    else:
        raise ValueError(op)
    dy = normal(rng, (M, N), 0.0, 1.0)
    return {"x": to_storage(x, dtype), "gamma": to_storage(gamma, dtype), "beta": None,
            "dy": to_storage(dy, dtype)}


def gen_ln_stress(seed: int, M: int, N: int, dtype: str, row_frac: float = 0.1,
                  chan_frac: float = 0.001, big_mean: float = 1000.0,
                  big_sd: float = 1e-2, outlier_scale: float = 100.0):
    """Large-mean rows plus outlier channels.

    x ~ N(0, 1) everywhere; then round(row_frac * M) seeded rows are replaced
    by big_mean + N(0, big_sd); then round(chan_frac * N) seeded channels
    (at least one) are multiplied by outlier_scale in every row.  The value is
    stored in the I/O dtype only after all of that.
    """
    rng = np.random.default_rng(seed)
    x = normal(rng, (M, N), 0.0, 1.0)
    n_rows = int(round(row_frac * M))
    rows = np.sort(rng.choice(M, size=n_rows, replace=False)) if n_rows else np.zeros(0, np.int64)
    if n_rows:
        x[rows] = normal(rng, (n_rows, N), big_mean, big_sd)
    n_ch = max(1, int(round(chan_frac * N)))
    chans = np.sort(rng.choice(N, size=n_ch, replace=False))
    x[:, chans] *= np.float32(outlier_scale)
    gamma = uniform(rng, (N,), 0.5, 1.5)
    beta = normal(rng, (N,), 0.0, 0.1)
    return {"x": to_storage(x, dtype), "gamma": to_storage(gamma, dtype),
            "beta": to_storage(beta, dtype), "big_rows": rows, "outlier_channels": chans}


def gen_ln_large_mean(seed: int, M: int, N: int, dtype: str = "f32"):
    """Every row 1000 + N(0, 1e-2), no outliers: the cancellation stress."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (M, N), 1000.0, 1e-2)
    gamma = uniform(rng, (N,), 0.5, 1.5)
    beta = normal(rng, (N,), 0.0, 0.1)
    return {"x": to_storage(x, dtype), "gamma": to_storage(gamma, dtype),
            "beta": to_storage(beta, dtype)}


def check_row_f32() -> np.ndarray:
    """The ten values 1000.001, 1000.002, ..., 1000.010 as a [1, 10] float32 row
    (each decimal literal rounded to the nearest float32)."""
    vals = [float("1000.%03d" % k) for k in range(1, 11)]
    return np.array(vals, dtype=np.float64).astype(np.float32).reshape(1, 10)


# --------------------------------------------------------------------------
# the five measured configurations, and the residual-add follow-on
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    op: str          # "ln", "rms", "add_rms" (residual add, then RMSNorm), "rms_fp8",
                     # "ln_bwd", "rms_bwd" (backward from the forward's statistics)
    dtype: str       # "f32", "bf16", "f16"
    M: int
    N: int
    eps: float
    seed: int
    recipe: str
    scale: float = 1.0   # FP8 output: the static scale

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def ideal_bytes(self, with_stats: bool = True) -> int:
        """Bytes the method must move: x read once, y written once, gamma
        (and beta for LN) read once, fp32 mean+rstd (LN) or rstd (RMS); with
        the residual add also the residual read once and the sum written once.
        Backward: dy and x read once, dx written once, gamma read once, the
        stored statistics read once, fp32 dgamma (LayerNorm: and dbeta)
        written once."""
        e = self.elem_bytes
        if self.op in ("ln_bwd", "rms_bwd"):
            # dy and x read, dx written, gamma read, fp32 dgamma (and dbeta) written
            ln = self.op == "ln_bwd"
            b = 3 * self.M * self.N * e + self.N * e + self.N * 4 * (2 if ln else 1)
            if with_stats:
                b += self.M * (8 if ln else 4)
            return b
        if self.op == "rms_fp8":
            b = self.M * self.N * (e + 1)          # x read, one byte per code written
        else:
            b = (4 if self.op == "add_rms" else 2) * self.M * self.N * e
        b += self.N * e * (2 if self.op == "ln" else 1)
        if with_stats:
            b += self.M * (8 if self.op == "ln" else 4)
        return b


CONFIGS = {
    "ln_f32_128x1024": Workload(
        "ln_f32_128x1024", "ln", "f32", 128, 1024, 1e-5, 1001,
        "x~N(0,1), gamma~U(0.5,1.5), beta~N(0,0.1); plus the 10-value check row"),
    "rms_f32_8192x4096": Workload(
        "rms_f32_8192x4096", "rms", "f32", 8192, 4096, 1e-6, 1002,
        "x~U(-1,1), weight~U(0,1)"),
    "ln_bf16_16384x8192": Workload(
        "ln_bf16_16384x8192", "ln", "bf16", 16384, 8192, 1e-5, 1003,
        "x~N(0,1); 10% rows 1000+N(0,1e-2); 0.1% channels x100; gamma~U(0.5,1.5), beta~N(0,0.1)"),
    "rms_f32_65536x2048": Workload(
        "rms_f32_65536x2048", "rms", "f32", 65536, 2048, 1e-6, 1004,
        "x~U(-1,1), weight~U(0,1)"),
    "rms_bf16_65536x2048": Workload(
        "rms_bf16_65536x2048", "rms", "bf16", 65536, 2048, 1e-6, 1004,
        "x~U(-1,1), weight~U(0,1) (same draws as the fp32 variant, stored as bf16)"),
    "ln_bf16_4096x5120": Workload(
        "ln_bf16_4096x5120", "ln", "bf16", 4096, 5120, 1e-5, 1005,
        "x~N(3,2), gamma~U(0.5,1.5), beta~N(0,0.1)"),
    "ln_bf16_64x1048576": Workload(
        "ln_bf16_64x1048576", "ln", "bf16", 64, 1048576, 1e-5, 1005,
        "x~N(3,2), gamma~U(0.5,1.5), beta~N(0,0.1); second draw of seed 1005"),
    "add_rms_bf16_16384x8192": Workload(
        "add_rms_bf16_16384x8192", "add_rms", "bf16", 16384, 8192, 1e-6, 1006,
        "x~U(-1,1), residual~N(0,1), weight~U(0,1); residual add then RMSNorm"),
    "rms_fp8_bf16_16384x8192": Workload(
        "rms_fp8_bf16_16384x8192", "rms_fp8", "bf16", 16384, 8192, 1e-6, 1007,
        "x~U(-1,1), weight~U(0,1); RMSNorm with FP8 E4M3 output of y / (1/64)", 1.0 / 64),
    "ln_bwd_bf16_16384x8192": Workload(
        "ln_bwd_bf16_16384x8192", "ln_bwd", "bf16", 16384, 8192, 1e-5, 1008,
        "x~N(0,1), gamma~U(0.5,1.5), dy~N(0,1); mean/rstd from the forward; LayerNorm backward"),
    "rms_bwd_bf16_16384x8192": Workload(
        "rms_bwd_bf16_16384x8192", "rms_bwd", "bf16", 16384, 8192, 1e-6, 1009,
        "x~U(-1,1), weight~U(0,1), dy~N(0,1); rstd from the forward; RMSNorm backward"),
    "ln_bwd_bf16_4096x32768": Workload(
        "ln_bwd_bf16_4096x32768", "ln_bwd", "bf16", 4096, 32768, 1e-5, 1010,
        "x~N(0,1), gamma~U(0.5,1.5), dy~N(0,1); LayerNorm backward on the longest rows of the row kernel"),
    "ln_bwd_bf16_64x1048576": Workload(
        "ln_bwd_bf16_64x1048576", "ln_bwd", "bf16", 64, 1048576, 1e-5, 1011,
        "x~N(0,1), gamma~U(0.5,1.5), dy~N(0,1); LayerNorm backward on rows split across workgroups"),
}


def generate(name: str) -> dict:
    """Inputs of a named configuration at full size."""
    w = CONFIGS[name]
    if name == "ln_f32_128x1024":
        return gen_ln_normal(w.seed, w.M, w.N, w.dtype)
    if name in ("rms_f32_8192x4096", "rms_f32_65536x2048", "rms_bf16_65536x2048"):
        return gen_rms_uniform(w.seed, w.M, w.N, w.dtype)
    if name == "ln_bf16_16384x8192":
        return gen_ln_stress(w.seed, w.M, w.N, w.dtype)
    if name == "ln_bf16_4096x5120":
        return gen_ln_normal(w.seed, w.M, w.N, w.dtype, loc=3.0, scale=2.0)
    if name == "ln_bf16_64x1048576":
        rng = np.random.default_rng(w.seed)
        a = CONFIGS["ln_bf16_4096x5120"]
        gen_ln_normal(0, a.M, a.N, a.dtype, loc=3.0, scale=2.0, rng=rng)   # first draw
        return gen_ln_normal(0, w.M, w.N, w.dtype, loc=3.0, scale=2.0, rng=rng)
    if name == "add_rms_bf16_16384x8192":
        return gen_add_rms(w.seed, w.M, w.N, w.dtype)
    if name == "rms_fp8_bf16_16384x8192":
        return gen_rms_uniform(w.seed, w.M, w.N, w.dtype)
    if w.op in ("ln_bwd", "rms_bwd"):
        return gen_bwd(w.seed, w.M, w.N, w.dtype, w.op)
    raise KeyError(name)
