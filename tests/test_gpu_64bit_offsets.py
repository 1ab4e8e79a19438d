"""Calls over more than 2^31 elements: element offsets past 32 bits, on the
row kernel (N = 8192, 262200 rows) and on the split rows (N = 2^20, 2049
rows, many batches), forward and backward, through the C ABI.

The matrices are 4.3 GB each, too large to draw on the host within a test's
time, so they are drawn on the device by torch's seeded generator.  The
oracle gets host copies of exactly those inputs, for sampled rows on both
sides of the 2^31-element boundary and the last rows (y, mean, rstd, dx).
For the column sums it gets sampled columns, every row. The backward's fp32
statistics come from torch in float64 (rounded to fp32), not from the
library.
"""
from __future__ import annotations

import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import oracle  # noqa: E402
import parity  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
rn = pytest.importorskip("rmsnorm_forward_amd")

TWO31 = 1 << 31
ROWS_CASES = [(262_200, 8192), (2049, 1 << 20)]   # row kernel, split rows


def normal(shape, seed, loc=0.0, scale=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16) * scale + loc


def uniform(n, seed, lo, hi):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.rand(n, generator=g, device="cuda", dtype=torch.float32) * (hi - lo) + lo).to(torch.bfloat16)


def host(t):
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def rows_across(M, N, seed, n=24):
    """Rows around the 2^31-element boundary, the first and last rows, and a
    random sample past the boundary."""
    b = TWO31 // N
    assert 0 < b < M
    rng = np.random.default_rng(seed)
    rows = {0, 1, b - 1, b, min(b + 1, M - 1), M - 2, M - 1}
    rows |= set(rng.integers(b, M, size=n).tolist())
    return np.array(sorted(rows))


def cols_sample(N, seed, n=12):
    rng = np.random.default_rng(seed)
    return np.array(sorted({0, 1, N - 2, N - 1} | set(rng.integers(0, N, size=n).tolist())))


def path_of(desc):
    return dict(kv.split("=") for kv in desc.split())["path"]


def stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("M,N", ROWS_CASES)
def test_ln_fwd_past_2_31_elements(M, N):
    assert M * N > TWO31
    want = "rows" if N == 8192 else "split"
    assert path_of(rn.norm_describe("ln", M, N, "bf16")).startswith(want)
    print(f"[gpu] ln_fwd bf16 M={M} N={N} ({M * N} elements)", flush=True)
    x = normal((M, N), 11, loc=3.0, scale=2.0)
    g = uniform(N, 12, 0.5, 1.5)
    b = normal((N,), 13, scale=0.1)
    y = torch.empty_like(x)
    mean = torch.empty(M, device="cuda")
    rstd = torch.empty(M, device="cuda")
    st = rn.ln_fwd(x.data_ptr(), g.data_ptr(), b.data_ptr(), y.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                   M, N, 1e-5, rn.NORM_BF16, stream())
    assert st == rn.NORM_OK, rn.norm_status_str(st)
    torch.cuda.synchronize()
    rows = rows_across(M, N, M)
    idx = torch.as_tensor(rows, device="cuda")
    yr, mr, rr = oracle.ln_fwd(host(x[idx]), host(g), host(b), "bf16", 1e-5)
    what = f"ln_fwd {M}x{N}"
    parity.check_y(host(y[idx]), yr, "bf16", what)
    parity.check_stats(host(mean[idx]), host(rstd[idx]), mr, rr, 1e-5, what)
    del x, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,N", ROWS_CASES)
def test_add_rms_fwd_past_2_31_elements(M, N):
    print(f"[gpu] add_rms_fwd bf16 M={M} N={N} ({M * N} elements)", flush=True)
    x = normal((M, N), 21)
    res = normal((M, N), 22)
    g = uniform(N, 23, 0.0, 1.0)
    y = torch.empty_like(x)
    h = torch.empty_like(x)
    rstd = torch.empty(M, device="cuda")
    st = rn.add_rms_fwd(x.data_ptr(), res.data_ptr(), g.data_ptr(), y.data_ptr(), h.data_ptr(), rstd.data_ptr(),
                        M, N, 1e-6, rn.NORM_BF16, stream())
    assert st == rn.NORM_OK, rn.norm_status_str(st)
    torch.cuda.synchronize()
    rows = rows_across(M, N, M + 1)
    idx = torch.as_tensor(rows, device="cuda")
    hr, yr, rr = oracle.add_rms_fwd(host(x[idx]), host(res[idx]), host(g), "bf16", 1e-6)
    what = f"add_rms_fwd {M}x{N}"
    assert np.array_equal(host(h[idx]), hr), f"{what}: residual sum differs from the oracle"
    parity.check_y(host(y[idx]), yr, "bf16", what)
    parity.check_stats(None, host(rstd[idx]), None, rr, 1e-6, what)
    del x, res, y, h
    torch.cuda.empty_cache()


def stats_f64(op, x, eps, chunk_elems=1 << 27):
    """Per-row mean and rstd by torch in float64, rounded to fp32."""
    M, N = x.shape
    mean = torch.empty(M, device="cuda")
    rstd = torch.empty(M, device="cuda")
    ch = max(1, chunk_elems // N)
    for r0 in range(0, M, ch):
        xs = x[r0:r0 + ch].double()
        if op == "ln":
            var, mu = torch.var_mean(xs, dim=1, unbiased=False)
            mean[r0:r0 + ch] = mu.float()
        else:
            var = (xs * xs).mean(1)
        rstd[r0:r0 + ch] = torch.rsqrt(var + eps).float()
    return mean, rstd


@pytest.mark.parametrize("op,M,N", [("ln", 262_200, 8192), ("rms", 2049, 1 << 20), ("ln", 2049, 1 << 20),
                                    ("rms", 262_200, 8192)])
def test_bwd_past_2_31_elements(op, M, N):
    eps = 1e-5 if op == "ln" else 1e-6
    desc = rn.norm_bwd_describe(op, M, N, "bf16", True)
    plan = {k: (v if k in ("path", "op", "mode") else int(v)) for k, v in (kv.split("=") for kv in desc.split())}
    print(f"[gpu] {op}_bwd bf16 M={M} N={N} ({M * N} elements) {desc}", flush=True)
    dy = normal((M, N), 31)
    x = normal((M, N), 32)
    g = uniform(N, 33, 0.5, 1.5)
    mean, rstd = stats_f64(op, x, eps)
    dx = torch.empty_like(x)
    dg = torch.empty(N, device="cuda")
    db = torch.empty(N, device="cuda")
    if op == "ln":
        st = rn.ln_bwd(dy.data_ptr(), x.data_ptr(), g.data_ptr(), mean.data_ptr(), rstd.data_ptr(), dx.data_ptr(),
                       dg.data_ptr(), db.data_ptr(), M, N, rn.NORM_BF16, stream())
    else:
        st = rn.rms_bwd(dy.data_ptr(), x.data_ptr(), g.data_ptr(), rstd.data_ptr(), dx.data_ptr(), dg.data_ptr(),
                        M, N, rn.NORM_BF16, stream())
    assert st == rn.NORM_OK, rn.norm_status_str(st)
    torch.cuda.synchronize()
    what = f"{op}_bwd {M}x{N}"
    mean_h = host(mean).astype(np.float64)
    rstd_h = host(rstd).astype(np.float64)
    gh = host(g)

    # dx on sampled rows (each row's dx depends on that row only)
    rows = rows_across(M, N, M + 2)
    idx = torch.as_tensor(rows, device="cuda")
    parity.check_bwd(op, "bf16", host(dy[idx]), host(x[idx]), gh, mean_h[rows] if op == "ln" else None,
                     rstd_h[rows], host(dx[idx]), None, None, None, what=what)

    # dgamma / dbeta on sampled columns, every row
    cols = cols_sample(N, N)
    cidx = torch.as_tensor(cols, device="cuda")
    dyc, xc = host(dy[:, cidx]), host(x[:, cidx])
    dys, xs = oracle.widen(dyc, "bf16"), oracle.widen(xc, "bf16")
    if op == "ln":
        ref = oracle.ln_bwd(dyc, xc, gh[cols], "bf16", mean_h, rstd_h)
        xh = (xs - mean_h[:, None]) * rstd_h[:, None]
        pairs = [(host(dg)[cols], ref[1], np.abs(dys * xh).sum(0), "dgamma"),
                 (host(db)[cols], ref[2], np.abs(dys).sum(0), "dbeta")]
    else:
        ref = oracle.rms_bwd(dyc, xc, gh[cols], "bf16", rstd_h)
        pairs = [(host(dg)[cols], ref[1], np.abs(dys * xs * rstd_h[:, None]).sum(0), "dgamma")]
    n = parity.bwd_chain(plan, M) + 4
    for got, want, mag, name in pairs:
        tol = n * parity.U32 * mag
        err = np.abs(got.astype(np.float64) - want)
        bad = ~(err <= tol)
        assert not bad.any(), (f"{what} {name}[{cols[np.argmax(bad)]}]: gpu={got[np.argmax(bad)]!r} "
                               f"oracle={want[np.argmax(bad)]!r} tol={tol[np.argmax(bad)]:.3g}")
    del dy, x, dx
    torch.cuda.empty_cache()
