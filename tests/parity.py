"""GPU-vs-oracle comparison at the stated tolerances.

Tolerances (the stated accuracy target for the forward; the readings where it
is open are marked):
  fp32 y        max |y_gpu - y_oracle| <= 2e-5
  bf16/fp16 y   within one unit in the last place of the oracle's value
                rounded to the I/O dtype (round-to-nearest-even), where the
                unit is that of the rounded value's binade; reading: a floor
                of 2^-20 applies to values so small that fp32 rounding of
                order-one intermediate terms exceeds their own ulp
  mean          |mean_gpu - mean_oracle| <= 1e-5 * max(|mean|, sqrt(var + eps));
                reading: plain relative error is ill-conditioned for rows whose
                mean is near zero, so the row's scale bounds it from below
  rstd          relative error <= 1e-5
  stress rows   no NaN, no infinity, variance >= 0 (rstd <= 1/sqrt(eps))
  FP8 codes     equal to the oracle's code of y / scale; where the two differ
                they must be neighbours and the oracle's y / scale must lie
                within FP8_TIE_REL of the midpoint between them (the kernel
                takes the decision on its fp32 y, which carries a few fp32
                ulps: reading), at most FP8_TIE_FRAC of all elements; a
                zero may be coded +0 or -0, a NaN with either sign

Backward (ln_bwd / rms_bwd; reading: no tolerance is stated for it, so
the bound is derived from the kernel's fp32 arithmetic, u = 2^-24, on the
same fp32 mean / rstd the oracle is given):
  dx            |dx_gpu - dx_oracle| <= B + (half an ulp of the I/O dtype at
                |dx_oracle| + B; none for fp32) with, per element,
                  LayerNorm  B = K u rstd (|g| + mean|g| + |xhat| mean|g xhat|)
                  RMSNorm    B = K u (rstd |g| + |x| rstd^3 mean|g x|)
                g = dy gamma, means over the row, K = BWD_K: each term passes
                through at most 32 sequential lane additions, a 10-level
                team tree, the cross-wavefront sum and a handful of
                products, so K = 128 covers every rounding with room
  dgamma/dbeta  |err| <= (n + 4) u sum_r |term| where n is the longest
                chain of fp32 additions any column goes through (rows per
                team + teams per workgroup + partial rows per wavefront of
                the column sum + 16) and term = dy xhat (RMSNorm dy x rstd),
                or dy for dbeta
"""
from __future__ import annotations

import numpy as np

import oracle

Y_F32_ABS = 2e-5
STAT_REL = 1e-5
HALF_FLOOR = 2.0 ** -20
SIG_BITS = {"bf16": 8, "f16": 11}
FP8_TIE_REL = 4e-6
FP8_TIE_FRAC = 1e-3


def _e4m3_table() -> np.ndarray:
    v = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, f = (c >> 3) & 0xF, c & 7
        if e == 0xF and f == 7:
            v[c] = np.nan
        elif e == 0:
            v[c] = s * f / 8.0 * 2.0 ** -6
        else:
            v[c] = s * (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return v


E4M3 = _e4m3_table()


def check_fp8(q_gpu: np.ndarray, q_ref: np.ndarray, y_ref: np.ndarray, scale: float, what: str = "") -> dict:
    """q_gpu, q_ref: uint8 codes; y_ref: the oracle's float64 y (before
    quantisation)."""
    g = E4M3[q_gpu.astype(np.int64)]
    r = E4M3[q_ref.astype(np.int64)]
    same = (q_gpu == q_ref) | ((g == 0) & (r == 0)) | (np.isnan(g) & np.isnan(r))
    diff = ~same
    n_tie = int(diff.sum())
    if n_tie:
        v = y_ref[diff] / float(np.float32(scale))
        gd, rd = g[diff], r[diff]
        mid = (gd + rd) / 2
        finite = np.isfinite(gd) & np.isfinite(rd)
        # neighbours: nothing representable strictly between them
        lo, hi = np.minimum(gd, rd), np.maximum(gd, rd)
        fin = E4M3[np.isfinite(E4M3)]
        between = np.array([np.any((fin > a) & (fin < b)) for a, b in zip(lo, hi)]) if finite.any() else \
            np.zeros(0, bool)
        near = np.abs(v - mid) <= FP8_TIE_REL * np.abs(v) + 1e-30
        bad = ~(finite & ~between & near)
        if bad.any():
            i = np.flatnonzero(diff)[np.flatnonzero(bad)[0]]
            raise AssertionError(f"{what}: FP8 code {q_gpu.flat[i]:#x} vs oracle {q_ref.flat[i]:#x} "
                                 f"for y/scale={y_ref.flat[i] / float(np.float32(scale))!r}")
        assert n_tie <= FP8_TIE_FRAC * q_gpu.size + 1, f"{what}: {n_tie} near-tie differences"
    return {"fp8_near_ties": n_tie}


def ulp_of(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the I/O dtype at |v| (v already representable in it)."""
    p = SIG_BITS[dtype]
    emin = -126 if dtype == "bf16" else -14
    a = np.maximum(np.abs(v), 2.0 ** emin)
    return np.exp2(np.floor(np.log2(a)) - (p - 1))


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """y_gpu: storage array; y_ref: float64 oracle result (same shape)."""
    if dtype == "f32":
        err = np.abs(y_gpu.astype(np.float64) - y_ref)
        bad = ~(err <= Y_F32_ABS)
        stats = {"max_abs_err": float(np.nanmax(err)) if err.size else 0.0}
    else:
        want = oracle.widen(oracle.round_to(y_ref, dtype), dtype)
        got = oracle.widen(y_gpu, dtype)
        err = np.abs(got - want)
        tol = np.maximum(ulp_of(want, dtype), HALF_FLOOR)
        bad = ~(err <= tol)
        both_nan = np.isnan(got) & np.isnan(want)
        bad &= ~both_nan
        stats = {"max_ulp_err": float(np.nanmax(err / tol)) if err.size else 0.0,
                 "exact_frac": float(np.mean(err == 0)) if err.size else 1.0}
    if np.any(bad):
        idx = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError(f"{what} y mismatch at {idx}: gpu={np.asarray(y_gpu)[idx]!r} "
                             f"oracle={y_ref[idx]!r} ({int(bad.sum())} bad of {bad.size}); {stats}")
    return stats


def check_stats(mean_gpu, rstd_gpu, mean_ref, rstd_ref, eps: float, what: str = "") -> dict:
    e = oracle.eps_as_kernel_sees(eps)
    out = {}
    if rstd_gpu is not None:
        rel = np.abs(rstd_gpu.astype(np.float64) - rstd_ref) / np.abs(rstd_ref)
        if not np.all(rel <= STAT_REL):
            i = int(np.nanargmax(rel))
            raise AssertionError(f"{what} rstd row {i}: gpu={rstd_gpu[i]!r} oracle={rstd_ref[i]!r} rel={rel[i]:.3g}")
        out["rstd_max_rel"] = float(rel.max()) if rel.size else 0.0
    if mean_gpu is not None:
        var = 1.0 / rstd_ref ** 2 - e
        scale = np.maximum(np.abs(mean_ref), np.sqrt(np.maximum(var, 0.0) + e))
        err = np.abs(mean_gpu.astype(np.float64) - mean_ref) / scale
        if not np.all(err <= STAT_REL):
            i = int(np.nanargmax(err))
            raise AssertionError(f"{what} mean row {i}: gpu={mean_gpu[i]!r} oracle={mean_ref[i]!r} err={err[i]:.3g}")
        out["mean_max_scaled_err"] = float(err.max()) if err.size else 0.0
    return out


def check_stress_invariants(rstd_gpu, y_gpu, dtype: str, eps: float, what: str = ""):
    """No NaN/inf anywhere; rstd finite and <= 1/sqrt(eps) (i.e. variance >= 0)."""
    e = oracle.eps_as_kernel_sees(eps)
    r = rstd_gpu.astype(np.float64)
    assert np.all(np.isfinite(r)), f"{what}: non-finite rstd"
    assert np.all(r <= (1 + 1e-6) / np.sqrt(e)), f"{what}: rstd implies a negative variance"
    yv = y_gpu.astype(np.float64) if dtype == "f32" else oracle.widen(y_gpu, dtype)
    assert np.all(np.isfinite(yv)), f"{what}: non-finite y"


BWD_K = 128
U32 = 2.0 ** -24


def bwd_chain(plan: dict, M: int) -> int:
    """Longest chain of fp32 additions behind one dgamma / dbeta column."""
    if plan.get("path") == "bwd_split":
        # each partial row adds its rows of every batch in turn, then the
        # column sums add the partial rows (16 wavefronts, then their sum)
        P, B = plan["partial_rows"], plan["batch_rows"]
        batches = -(-M // B) if M else 0
        return batches * (-(-B // P) + 1) + -(-P // 16) + 16
    rows_per_team = -(-plan["work"] // plan["grid"]) if plan["grid"] else 0
    return rows_per_team + plan["rows_per_wg"] + -(-plan["grid"] // 16) + 16


def check_bwd(op: str, dtype: str, dy, x, gamma, mean, rstd, dx, dg, db, plan: dict | None, rows=None,
              what: str = "") -> dict:
    """dy, x, gamma: storage arrays; mean, rstd: the fp32 statistics given to
    both sides; dx (rows `rows` only when given), dg, db: the GPU's results
    (None = not checked).  dg / db need every row."""
    M, N = x.shape
    xs = oracle.widen(x, dtype)
    dys = oracle.widen(dy, dtype)
    gam = np.ones(N) if gamma is None else oracle.widen(gamma, dtype)
    rs = np.asarray(rstd, np.float64)
    out = {}
    sel = np.arange(M) if rows is None else np.asarray(rows)
    if op == "ln":
        mu = np.asarray(mean, np.float64)
        ref = oracle.ln_bwd(dy[sel], x[sel], gamma, dtype, mu[sel], rs[sel])
        dxr = ref[0]
        xh = (xs[sel] - mu[sel, None]) * rs[sel, None]
        g = dys[sel] * gam
        B = BWD_K * U32 * rs[sel, None] * (np.abs(g) + np.abs(g).mean(1, keepdims=True)
                                           + np.abs(xh) * np.abs(g * xh).mean(1, keepdims=True))
    else:
        ref = oracle.rms_bwd(dy[sel], x[sel], gamma, dtype, rs[sel])
        dxr = ref[0]
        g = dys[sel] * gam
        r = rs[sel, None]
        B = BWD_K * U32 * (r * np.abs(g) + np.abs(xs[sel]) * r ** 3 * np.abs(g * xs[sel]).mean(1, keepdims=True))
    got = dx.astype(np.float64) if dtype == "f32" else oracle.widen(dx, dtype)
    tol = B if dtype == "f32" else B + 0.5 * ulp_of(np.abs(dxr) + B, dtype)
    err = np.abs(got - dxr)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError(f"{what} dx mismatch at row {sel[i[0]]} col {i[1]}: gpu={got[i]!r} "
                             f"oracle={dxr[i]!r} tol={tol[i]:.3g} ({int(bad.sum())} bad of {bad.size})")
    out["dx_max_err_over_tol"] = float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0
    if dg is not None or db is not None:
        assert rows is None, "column sums need every row"
        n = bwd_chain(plan, M) + 4
        full = ref
        if op == "ln":
            xh_all = (xs - np.asarray(mean, np.float64)[:, None]) * rs[:, None]
            pairs = [(dg, full[1], np.abs(dys * xh_all).sum(0), "dgamma"),
                     (db, full[2], np.abs(dys).sum(0), "dbeta")]
        else:
            pairs = [(dg, full[1], np.abs(dys * xs * rs[:, None]).sum(0), "dgamma")]
        for got_c, want_c, mag, name in pairs:
            if got_c is None:
                continue
            tol_c = n * U32 * mag
            e = np.abs(got_c.astype(np.float64) - want_c)
            badc = ~(e <= tol_c)
            if badc.any():
                j = int(np.argmax(badc))
                raise AssertionError(f"{what} {name}[{j}]: gpu={got_c[j]!r} oracle={want_c[j]!r} "
                                     f"tol={tol_c[j]:.3g} ({int(badc.sum())} bad of {badc.size})")
            out[f"{name}_max_err_over_tol"] = float((e / np.maximum(tol_c, 1e-300)).max()) if e.size else 0.0
    return out
