"""HIP path vs the CPU oracle, element by element, through the C ABI.

Shapes: every measured configuration at full size (sampled rows checked
against the oracle, properties checked on every row), plus small shapes that
span several tiles with ragged tails, the degenerate cases (N = 1, constant
rows, eps = 0, M = 0), unaligned pointers, every forced path and tile, and
bitwise determinism.
"""
from __future__ import annotations

import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import oracle  # noqa: E402
import parity  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
gpu_runner = pytest.importorskip("gpu_runner")
run = gpu_runner.run


def oracle_for(op, dtype, x, gamma, beta, eps):
    if op == "ln":
        return oracle.ln_fwd(x, gamma, beta, dtype, eps)
    y, r = oracle.rms_fwd(x, gamma, dtype, eps)
    return y, None, r


def compare(op, dtype, x, gamma, beta, eps, y, mean, rstd, rows=None, what=""):
    xs = x if rows is None else x[rows]
    yr, mr, rr = oracle_for(op, dtype, xs, gamma, beta if op == "ln" else None, eps)
    ys = y if rows is None else y[rows]
    out = parity.check_y(ys, yr, dtype, what)
    ms = None if mean is None else (mean if rows is None else mean[rows])
    rsv = None if rstd is None else (rstd if rows is None else rstd[rows])
    out.update(parity.check_stats(ms, rsv, mr, rr, eps, what))
    return out


def compare_add(dtype, x, res, gamma, eps, y, h, rstd, rows=None, what=""):
    """Residual add + RMSNorm: the stored sum h bit for bit, y and rstd to
    the same bar as rms_fwd."""
    xs = x if rows is None else x[rows]
    rs = res if rows is None else res[rows]
    hr, yr, rr = oracle.add_rms_fwd(xs, rs, gamma, dtype, eps)
    hs = h if rows is None else h[rows]
    bad = hs.view(np.uint8).reshape(hs.shape[0], -1) != hr.view(np.uint8).reshape(hr.shape[0], -1)
    assert not bad.any(), f"{what}: residual sum differs from the oracle at {np.argwhere(bad)[:4].tolist()}"
    ys = y if rows is None else y[rows]
    out = parity.check_y(ys, yr, dtype, what)
    if rstd is not None:
        out.update(parity.check_stats(None, rstd if rows is None else rstd[rows], None, rr, eps, what))
    return out


def sample_rows(M, n=256, seed=0, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(range(min(4, M))) | set(range(max(0, M - 4), M)) | set(extra)
    rows |= set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(rows))


# ---------------------------------------------------------------------------
# measured configurations at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_measured_configuration(name):
    w = workloads.CONFIGS[name]
    print(f"[gpu] config {name}: {w.op} {w.dtype} M={w.M} N={w.N}", flush=True)
    inp = workloads.generate(name)
    if w.op == "rms_fp8":
        q, _, rstd = gpu_runner.run_fp8(w.dtype, inp["x"], None, inp["gamma"], w.eps, w.scale)
        rows = sample_rows(w.M, 256, seed=w.seed)
        qr, yr, rr = oracle.rms_fp8_fwd(inp["x"][rows], inp["gamma"], w.dtype, w.eps, w.scale)
        st = parity.check_fp8(q[rows], qr, yr, w.scale, name)
        st.update(parity.check_stats(None, rstd[rows], None, rr, w.eps, name))
        print(f"[gpu] {name}: {st}", flush=True)
        return
    if w.op == "add_rms":
        y, h, rstd = gpu_runner.run_add(w.dtype, inp["x"], inp["res"], inp["gamma"], w.eps)
        rows = sample_rows(w.M, 256, seed=w.seed)
        st = compare_add(w.dtype, inp["x"], inp["res"], inp["gamma"], w.eps, y, h, rstd, rows, name)
        parity.check_stress_invariants(rstd, y, w.dtype, w.eps, name)
        print(f"[gpu] {name}: {st}", flush=True)
        return
    y, mean, rstd = run(w.op, w.dtype, inp["x"], inp["gamma"], inp["beta"], w.eps)
    extra = ()
    if "big_rows" in inp:
        extra = inp["big_rows"][:512]
    rows = None if w.M * w.N <= (1 << 25) else sample_rows(w.M, 256, seed=w.seed, extra=extra)
    if w.N >= (1 << 20):
        rows = sample_rows(w.M, 6, seed=w.seed)
    st = compare(w.op, w.dtype, inp["x"], inp["gamma"], inp["beta"], w.eps, y, mean, rstd, rows, name)
    parity.check_stress_invariants(rstd, y, w.dtype, w.eps, name)
    print(f"[gpu] {name}: {st}", flush=True)


def test_check_row_large_mean():
    """The 10-value row 1000.001..1000.010 as its own M=1, N=10 fp32 call with
    gamma = 1 and beta = 0 (NULL), eps = 1e-5."""
    x = workloads.check_row_f32()
    y, mean, rstd = run("ln", "f32", x, None, None, 1e-5)
    st = compare("ln", "f32", x, None, None, 1e-5, y, mean, rstd, what="check row")
    assert st["max_abs_err"] <= 2e-5
    yr, mr, rr = oracle.ln_fwd(x, None, None, "f32", 1e-5)
    var_gpu = 1.0 / float(rstd[0]) ** 2 - oracle.eps_as_kernel_sees(1e-5)
    var_ref = 1.0 / rr[0] ** 2 - oracle.eps_as_kernel_sees(1e-5)
    assert abs(var_gpu - var_ref) <= 1e-4 * var_ref


# ---------------------------------------------------------------------------
# shapes across tiles, ragged tails, all dtypes, both ops
# ---------------------------------------------------------------------------

EDGE_N = [1, 2, 3, 5, 7, 8, 10, 16, 63, 64, 65, 127, 128, 1000, 1023, 1024, 1025,
          2047, 2048, 4096, 5120, 8191, 8192, 8193, 16384, 24576, 32768, 40000, 65536, 65544,
          131072, 131080]


def inputs(op, dtype, M, N, seed):
    if op == "ln":
        return workloads.gen_ln_normal(seed, M, N, dtype, loc=3.0, scale=2.0)
    return workloads.gen_rms_uniform(seed, M, N, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["ln", "rms"])
@pytest.mark.parametrize("N", EDGE_N)
def test_edge_shapes(op, dtype, N):
    M = 37 if N <= 8192 else 5
    print(f"[gpu] edge {op} {dtype} M={M} N={N}", flush=True)
    inp = inputs(op, dtype, M, N, seed=N)
    y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what=f"N={N}")


@pytest.mark.parametrize("mode", ["split2", "splitpass"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("op", ["ln", "rms"])
@pytest.mark.parametrize("N", [10, 1000, 8192, 65544, 300000])
def test_forced_split_path(monkeypatch, op, dtype, N, mode):
    monkeypatch.setenv("MI355NORM_PATH", mode)
    M = 9
    print(f"[gpu] {mode} {op} {dtype} M={M} N={N}", flush=True)
    inp = inputs(op, dtype, M, N, seed=N + 1)
    y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what=f"split N={N}")


TILES = [(t, v) for t in (4, 8, 16, 32, 64, 128, 256, 512, 1024) for v in (1, 2, 4, 8, 16)] + [(64, 5), (64, 10)]


@pytest.mark.parametrize("dtype,N", [("bf16", 4096), ("f32", 1000), ("f16", 2056)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_every_tile(monkeypatch, op, dtype, N):
    """Every instantiated tile that covers the row gives oracle-exact results."""
    M = 19
    inp = inputs(op, dtype, M, N, seed=17)
    e = 4 if dtype == "f32" else 2
    epv = 16 // e if (N * e) % 16 == 0 else 1
    nv = N // epv
    ran = 0
    for t, v in TILES:
        if t * v < nv:
            continue
        monkeypatch.setenv("MI355NORM_TILE", f"{t}x{v}")
        print(f"[gpu] tile {t}x{v} {op} {dtype} N={N}", flush=True)
        y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
        compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what=f"tile {t}x{v}")
        ran += 1
    assert ran >= 5


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_unaligned_pointers(op, dtype):
    """Pointers one element past a 16-byte boundary take the element-wise path."""
    M, N = 23, 4096
    inp = inputs(op, dtype, M, N, seed=5)
    y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, offset=1)
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what="unaligned")


@pytest.mark.parametrize("op,dtype,M,N,tile", [("rms", "bf16", 64, 8192, "512x2"), ("rms", "f16", 37, 6144, "512x2"),
                                               ("rms", "bf16", 16, 16384, "1024x2"),
                                               ("rms_fp8", "bf16", 9, 12288, "256x8"),
                                               ("rms_fp8", "f32", 9, 8192, "256x8"),
                                               ("rms_fp8", "bf16", 5, 32768, "512x8")])
def test_long_rms_row_tiles(op, dtype, M, N, tile):
    """The tiles the planner picks for long RMSNorm rows (two vectors per
    lane with 16-bit I/O, eight with FP8 output), against the oracle."""
    import rmsnorm_forward_amd as rn
    d = dict(kv.split("=") for kv in rn.norm_describe(op, M, N, dtype).split())
    assert f"{d['team']}x{d['vpl']}" == tile, d
    print(f"[gpu] long rms rows {op} {dtype} {M}x{N} tile {tile}", flush=True)
    inp = inputs("rms", dtype, M, N, seed=N + 41)
    if op == "rms":
        y, _, rstd = run("rms", dtype, inp["x"], inp["gamma"], None, 1e-6)
        compare("rms", dtype, inp["x"], inp["gamma"], None, 1e-6, y, None, rstd, what=f"rms {tile}")
    else:
        q, _, r = gpu_runner.run_fp8(dtype, inp["x"], None, inp["gamma"], 1e-6, 0.05)
        compare_fp8(dtype, inp["x"], None, inp["gamma"], 1e-6, 0.05, q, None, r, what=f"fp8 {tile}")


@pytest.mark.parametrize("dtype,N", [("bf16", 5120), ("bf16", 2560), ("f32", 2560), ("f32", 1280), ("f16", 5120)])
@pytest.mark.parametrize("M", [1, 1001, 4096])
def test_one_wavefront_tiles(M, dtype, N):
    """Rows of 320 or 640 16-byte vectors and at most 4096 rows take one
    wavefront per row with 5 or 10 vectors per lane: every operation against
    the oracle, ragged row counts included (4 rows per workgroup)."""
    import rmsnorm_forward_amd as rn
    e = 4 if dtype == "f32" else 2
    d = dict(kv.split("=") for kv in rn.norm_describe("ln", M, N, dtype).split())
    assert (d["team"], d["vpl"]) == ("64", str(N * e // 16 // 64)), d
    rows = None if M <= 1001 else sample_rows(M, 64, seed=N)
    what = f"one-wavefront {dtype} {M}x{N}"
    print(f"[gpu] {what}", flush=True)
    for op in ("ln", "rms"):
        inp = inputs(op, dtype, M, N, seed=M + N)
        y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
        compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, rows, what=f"{op} {what}")
    inp = workloads.gen_add_rms(M + N, M, N, dtype)
    y, h, rstd = gpu_runner.run_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6)
    compare_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, y, h, rstd, rows, what=f"add_rms {what}")
    if rows is None:
        for res in (None, inp["res"]):
            q, hq, rq = gpu_runner.run_fp8(dtype, inp["x"], res, inp["gamma"], 1e-6, 1.0 / 64)
            compare_fp8(dtype, inp["x"], res, inp["gamma"], 1e-6, 1.0 / 64, q, hq, rq,
                        what=f"fp8 add={res is not None} {what}")


@pytest.mark.parametrize("has_g,has_b", [(False, False), (True, False), (False, True)])
def test_optional_gamma_beta(has_g, has_b):
    M, N = 33, 3000
    inp = inputs("ln", "bf16", M, N, seed=21)
    g = inp["gamma"] if has_g else None
    b = inp["beta"] if has_b else None
    y, mean, rstd = run("ln", "bf16", inp["x"], g, b, 1e-5)
    compare("ln", "bf16", inp["x"], g, b, 1e-5, y, mean, rstd, what="optional gamma/beta")
    y2, m2, r2 = run("ln", "bf16", inp["x"], g, b, 1e-5, stats=False)
    assert np.array_equal(y, y2) and m2 is None and r2 is None


def test_rms_without_gamma_or_rstd():
    M, N = 40, 2048
    inp = inputs("rms", "f32", M, N, seed=22)
    y, _, rstd = run("rms", "f32", inp["x"], None, None, 1e-6)
    compare("rms", "f32", inp["x"], None, None, 1e-6, y, None, rstd, what="rms no gamma")
    y2, _, r2 = run("rms", "f32", inp["x"], None, None, 1e-6, stats=False)
    assert np.array_equal(y, y2) and r2 is None


@pytest.mark.parametrize("N", [1, 7, 4096])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_constant_rows(dtype, N):
    """Constant rows (and N = 1): y = beta exactly, mean = the constant,
    rstd = 1/sqrt(eps); with eps = 0, rstd = inf and y = NaN like the oracle."""
    M = 6
    x32 = np.repeat(np.array([0.0, 1.0, -3.5, 1000.0, 99840.0, 2.0 ** -10], np.float32)[:, None], N, axis=1)
    x = workloads.to_storage(x32, dtype)
    rng = np.random.default_rng(3)
    g = workloads.to_storage(rng.uniform(0.5, 1.5, N).astype(np.float32), dtype)
    b = workloads.to_storage(rng.normal(0, 0.1, N).astype(np.float32), dtype)
    y, mean, rstd = run("ln", dtype, x, g, b, 1e-5)
    assert np.array_equal(y, np.broadcast_to(b, y.shape))
    assert np.array_equal(mean.astype(np.float64), oracle.widen(x[:, 0], dtype))
    compare("ln", dtype, x, g, b, 1e-5, y, mean, rstd, what="constant rows")
    y0, mean0, rstd0 = run("ln", dtype, x, g, b, 0.0)
    assert np.all(np.isinf(rstd0))
    yv = y0.astype(np.float64) if dtype == "f32" else oracle.widen(y0, dtype)
    assert np.all(np.isnan(yv))


@pytest.mark.parametrize("mode", ["split2", "split1"])
@pytest.mark.parametrize("dtype,N", [("f32", 100000), ("bf16", 1 << 18)])
def test_constant_split_rows(monkeypatch, mode, dtype, N):
    """Constant rows split across workgroups, in both split forms: every
    chunk's partial has M2 = 0, so the merged variance is exactly 0, y is
    beta exactly, the mean is the constant and rstd = 1/sqrt(eps); with
    eps = 0, rstd = inf and y = NaN.  RMSNorm of a zero row with eps = 0:
    rstd = inf, y = NaN; of a constant row, the oracle's values."""
    monkeypatch.setenv("MI355NORM_PATH", mode)
    M = 6
    x32 = np.repeat(np.array([0.0, 1.0, -3.5, 1000.0, 99840.0, 2.0 ** -10], np.float32)[:, None], N, axis=1)
    x = workloads.to_storage(x32, dtype)
    rng = np.random.default_rng(5)
    g = workloads.to_storage(rng.uniform(0.5, 1.5, N).astype(np.float32), dtype)
    b = workloads.to_storage(rng.normal(0, 0.1, N).astype(np.float32), dtype)
    print(f"[gpu] constant split rows {mode} {dtype} N={N}", flush=True)
    y, mean, rstd = run("ln", dtype, x, g, b, 1e-5)
    assert np.array_equal(y, np.broadcast_to(b, y.shape))
    assert np.array_equal(mean.astype(np.float64), oracle.widen(x[:, 0], dtype))
    compare("ln", dtype, x, g, b, 1e-5, y, mean, rstd, what="constant split rows")
    y0, _, rstd0 = run("ln", dtype, x, g, b, 0.0)
    assert np.all(np.isinf(rstd0))
    assert np.all(np.isnan(y0.astype(np.float64) if dtype == "f32" else oracle.widen(y0, dtype)))
    yr, _, rr = run("rms", dtype, x, g, None, 1e-6)
    compare("rms", dtype, x, g, None, 1e-6, yr, None, rr, what="constant split rows, rms")
    yz, _, rz = run("rms", dtype, x[:1], g, None, 0.0)
    assert np.isinf(rz[0]) and np.all(np.isnan(yz.astype(np.float64) if dtype == "f32" else oracle.widen(yz, dtype)))


def test_rms_zero_row_eps0():
    x = np.zeros((3, 256), np.float32)
    y, _, rstd = run("rms", "f32", x, None, None, 0.0)
    assert np.all(np.isinf(rstd)) and np.all(np.isnan(y))


def test_fp32_large_mean_stress():
    """Every row 1000 + N(0, 1e-2) in fp32 at N = 8192: the naive E[x^2]-E[x]^2
    formula goes negative on such rows; here variance must stay >= 0 and
    every output within the fp32 tolerances of the oracle."""
    inp = workloads.gen_ln_large_mean(1006, 64, 8192, "f32")
    y, mean, rstd = run("ln", "f32", inp["x"], inp["gamma"], inp["beta"], 1e-5)
    parity.check_stress_invariants(rstd, y, "f32", 1e-5, "fp32 stress")
    compare("ln", "f32", inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what="fp32 stress")


def test_stress_rows_small_bf16():
    """The large-mean + outlier-channel recipe at a size the oracle checks fully."""
    inp = workloads.gen_ln_stress(77, 512, 8192, "bf16", chan_frac=0.002)
    y, mean, rstd = run("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5)
    parity.check_stress_invariants(rstd, y, "bf16", 1e-5, "bf16 stress")
    compare("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what="bf16 stress")


@pytest.mark.parametrize("path", ["auto", "split2", "splitpass"])
def test_bitwise_deterministic(monkeypatch, path):
    if path != "auto":
        monkeypatch.setenv("MI355NORM_PATH", path)
    inp = inputs("ln", "bf16", 300, 8192, seed=31)
    a = run("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5)
    b = run("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_split_statistics_shared_by_all_chunks():
    """All workgroups of a split row must normalise with the same mean and
    rstd: with x, gamma and beta periodic in the chunk length, every full
    chunk of a row holds the same data, so its output must be bitwise equal
    to every other full chunk's."""
    import rmsnorm_forward_amd as rn
    N = 300000
    d = dict(kv.split("=") for kv in rn.norm_describe("ln", 2, N, "bf16").split())
    assert d["path"] == "split"
    C = int(d["wg"]) * int(d["vpl"]) * int(d["epv"])     # elements per chunk
    base = inputs("ln", "bf16", 2, C, seed=41)
    reps = -(-N // C)
    x = np.tile(base["x"], (1, reps))[:, :N].copy()
    g = np.tile(base["gamma"], reps)[:N].copy()
    b = np.tile(base["beta"], reps)[:N].copy()
    y, mean, rstd = run("ln", "bf16", x, g, b, 1e-5)
    full = N // C
    for r in range(2):
        for c in range(1, full):
            assert np.array_equal(y[r, :C], y[r, c * C:(c + 1) * C]), (r, c)
    compare("ln", "bf16", x, g, b, 1e-5, y, mean, rstd, what="periodic split")


def test_two_kernel_split_is_the_default_and_agrees_with_the_single_pass(monkeypatch):
    """The long-row configuration runs the two-kernel split by default.  The
    two kernels and the single pass (different chunk sizes, so different
    partials) both meet the oracle's bar, and their statistics agree to fp32
    rounding."""
    import rmsnorm_forward_amd as rn
    d = dict(kv.split("=") for kv in rn.norm_describe("ln", 64, 1 << 20, "bf16").split())
    assert d["path"] == "split" and d["mode"] == "two", d
    inp = inputs("ln", "bf16", 40, 1 << 18, seed=61)
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    a = run("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5)
    monkeypatch.setenv("MI355NORM_PATH", "split2")
    b = run("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5)
    monkeypatch.delenv("MI355NORM_PATH")
    compare("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5, *a, what="single pass")
    compare("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5, *b, what="two-kernel")
    assert np.max(np.abs(a[2] / b[2] - 1)) < 1e-5 and np.max(np.abs(a[1] - b[1])) < 1e-4


@pytest.mark.parametrize("dtype,N,offset", [("bf16", 140000, 0), ("f32", 70000, 0), ("f16", 20000, 1)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_row_batches(monkeypatch, op, dtype, N, offset):
    """The two kernels run rows split across workgroups in batches (here 3
    rows, so batches of 3, 3 and 1): every batch's rows, means and rstds land
    at their own offsets and meet the oracle's bar."""
    e = 4 if dtype == "f32" else 2
    monkeypatch.setenv("MI355NORM_PATH", "split2")
    monkeypatch.setenv("MI355NORM_SPLIT_BATCH", str(3 * N * e))
    M = 7
    print(f"[gpu] split batches {op} {dtype} M={M} N={N} offset={offset}", flush=True)
    inp = inputs(op, dtype, M, N, seed=N + 3)
    y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, offset=offset)
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what=f"batches N={N}")


@pytest.mark.parametrize("mode", ["split2", "splitpass"])
def test_split_workspace_reused_across_shapes(monkeypatch, mode):
    """Split calls of different shapes back to back on one stream share the
    kept workspace; each must see its counters at zero (a regression test:
    counters placed after shape-dependent partials once started a call
    non-zero and let a workgroup read partials early)."""
    monkeypatch.setenv("MI355NORM_PATH", mode)
    shapes = [(9, 300000), (5, 131080), (3, 1 << 18), (11, 140000), (2, 131080), (7, 65544 * 3)]
    for i, (M, N) in enumerate(shapes):
        for op in ("ln", "rms"):
            inp = inputs(op, "f32", M, N, seed=70 + i)
            y, mean, rstd = run(op, "f32", inp["x"], inp["gamma"], inp["beta"], 1e-5)
            compare(op, "f32", inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd,
                    what=f"reuse {mode} {op} M={M} N={N}")


# RMSNorm on 16-byte vectors: 16 wide chunks a row (bf16) and 8 chunks of
# 512 lanes (f16), whose one-reduction partials the recompute runs back to back
@pytest.mark.parametrize("op,dtype,M,N,offset", [("ln", "bf16", 6, 1 << 18, 0), ("rms", "f32", 5, 100003, 1),
                                                  ("ln", "f16", 40, 70000, 0), ("ln", "f32", 33, 65544, 0),
                                                  ("rms", "bf16", 8, 1 << 20, 0), ("rms", "f16", 6, 1 << 18, 0)])
def test_single_pass_recompute_gives_the_same_bits(monkeypatch, op, dtype, M, N, offset):
    """The single pass's bounded wait, forced from the host to give up at
    once: every workgroup then computes all of its rows' partials from x
    itself.  The outputs must be the bits of the normal single pass, and the
    kept workspace (slots, departure counters) must be back at zero for the
    next call, which must give those bits again."""
    monkeypatch.setenv("MI355NORM_PATH", "split1")
    inp = inputs(op, dtype, M, N, seed=62 + M)
    print(f"[gpu] single pass {op} {dtype} M={M} N={N} offset={offset}: normal, recompute, normal", flush=True)
    a = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, offset=offset)
    monkeypatch.setenv("MI355NORM_FORCE_TIMEOUT", "1")
    b = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, offset=offset)
    monkeypatch.delenv("MI355NORM_FORCE_TIMEOUT")
    c = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, offset=offset)
    for u, v, w in zip(a, b, c):
        if u is None:
            continue
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "recompute path differs"
        assert np.array_equal(u.view(np.uint8), w.view(np.uint8)), "call after the recompute differs"
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, *a, what="single pass")


@pytest.mark.parametrize("op,dtype,M,N", [("ln", "bf16", 200, 1 << 18), ("rms", "f32", 150, 131080),
                                           ("ln", "f16", 230, 131080)])
def test_single_pass_teams_walk_several_rows(monkeypatch, op, dtype, M, N):
    """More rows than teams of resident workgroups: each team walks several
    rows, and from its second row on every workgroup normalises the chunk it
    loaded into LDS while waiting on the previous row.  The normal run and a
    run forced onto the recomputation path must give the same bits, and both
    the oracle's values."""
    import rmsnorm_forward_amd as rn
    monkeypatch.setenv("MI355NORM_PATH", "split1")
    plan = dict(kv.split("=") for kv in rn.norm_describe(op, M, N, dtype).split())
    assert plan["mode"] == "pass" and int(plan["teams"]) < M, plan
    inp = inputs(op, dtype, M, N, seed=90 + M)
    print(f"[gpu] single pass, {plan['teams']} teams over {M} rows: {op} {dtype} N={N}", flush=True)
    a = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    monkeypatch.setenv("MI355NORM_FORCE_TIMEOUT", "1")
    b = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    monkeypatch.delenv("MI355NORM_FORCE_TIMEOUT")
    for u, v in zip(a, b):
        if u is not None:
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "recompute path differs"
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, *a, what="single pass, several rows per team")


@pytest.mark.parametrize("op,dtype,M,N", [("rms", "bf16", 40, 1 << 20), ("rms", "f16", 20, (1 << 20) + 8),
                                           ("rms", "f32", 20, (1 << 19) + 4), ("ln", "f32", 10, 1 << 20),
                                           ("rms_fp8", "bf16", 20, (1 << 20) + 8), ("rms_fp8", "f32", 18, 1 << 19)])
def test_single_pass_wide_chunks(monkeypatch, op, dtype, M, N):
    """Rows of at least 16 chunks of 1024 lanes x 8 vectors take those wide
    chunks in the single pass (RMSNorm, its FP8 output, fp32 LayerNorm):
    teams walk several rows, a ragged row's last chunk holds one vector, a
    run forced onto the recomputation path gives the same bits, and both
    give the oracle's values."""
    import rmsnorm_forward_amd as rn
    plan = dict(kv.split("=") for kv in rn.norm_describe(op, M, N, dtype).split())
    assert plan["mode"] == "pass" and plan["wg"] == "1024" and int(plan["teams"]) < M, plan
    inp = inputs("ln" if op == "ln" else "rms", dtype, M, N, seed=95 + M)
    print(f"[gpu] wide single pass {op} {dtype} M={M} N={N}: {plan['chunks']} chunks, {plan['teams']} teams",
          flush=True)
    if op == "rms_fp8":
        go = lambda: gpu_runner.run_fp8(dtype, inp["x"], None, inp["gamma"], 1e-6, 0.05)
    else:
        go = lambda: run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    a = go()
    monkeypatch.setenv("MI355NORM_FORCE_TIMEOUT", "1")
    b = go()
    monkeypatch.delenv("MI355NORM_FORCE_TIMEOUT")
    for u, v in zip(a, b):
        if u is not None:
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "recompute path differs"
    if op == "rms_fp8":
        compare_fp8(dtype, inp["x"], None, inp["gamma"], 1e-6, 0.05, a[0], None, a[2], what="wide single pass")
    else:
        compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, *a, what="wide single pass")


@pytest.mark.parametrize("mode", ["auto", "split2", "split1"])
@pytest.mark.parametrize("op,dtype,offset", [("ln", "bf16", 0), ("rms", "bf16", 0), ("rms", "f32", 0),
                                             ("ln", "f32", 1)])
def test_longest_rows(monkeypatch, op, dtype, offset, mode):
    """Rows of 2^24 elements, the longest the library takes, in every split
    form.  The single pass needs every chunk of a row resident at once: bf16
    rows of 16-byte vectors fit (RMSNorm: 256 chunks of 1024 lanes x 8
    vectors; LayerNorm: 512 of 512 lanes), fp32 rows (512 or 1024 chunks) and
    element-wise rows do not, so asking for it is refused before any launch,
    while the automatic choice falls back to the two kernels."""
    import rmsnorm_forward_amd as rn
    M, N = 2, 1 << 24
    aligned = offset == 0
    if mode != "auto":
        monkeypatch.setenv("MI355NORM_PATH", mode)
    if mode == "split1" and (dtype == "f32" or not aligned):
        with pytest.raises(RuntimeError):
            rn.norm_describe(op, M, N, dtype, aligned=aligned)
        return
    plan = dict(kv.split("=") for kv in rn.norm_describe(op, M, N, dtype, aligned=aligned).split())
    print(f"[gpu] longest rows {op} {dtype} offset={offset} {mode}: mode={plan['mode']} chunks={plan['chunks']}",
          flush=True)
    inp = inputs(op, dtype, M, N, seed=24 + offset)
    y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, offset=offset)
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what=f"N=2^24 {mode}")


def test_split_mode_chosen_automatically():
    """On the GPU, rows split across workgroups take the single pass for
    RMSNorm (plain and with FP8 output) and fp32 LayerNorm on 16-byte
    vectors, and for LayerNorm with 16-bit I/O when every team walks at most
    three rows; otherwise the two kernels, which the residual add and rows
    that are not 16-byte vectors always take."""
    import rmsnorm_forward_amd as rn
    N = 1 << 20
    mode = lambda op, dtype, aligned=True, M=64: dict(kv.split("=") for kv in
                                                      rn.norm_describe(op, M, N, dtype, aligned=aligned).split())["mode"]
    assert mode("rms", "bf16") == "pass" and mode("rms", "f32") == "pass" and mode("rms", "f16") == "pass"
    assert mode("rms_fp8", "bf16") == "pass"
    assert mode("ln", "f32") == "pass"
    assert mode("ln", "bf16") == "two" and mode("ln", "f16") == "two"          # 4 rows per team
    assert mode("ln", "bf16", M=16) == "pass" and mode("ln", "f16", M=48) == "pass"   # 1 and 3 rows per team
    assert mode("ln", "bf16", aligned=False, M=16) == "two"
    assert mode("add_rms", "bf16") == "two" and mode("add_rms", "f32") == "two"
    assert mode("rms", "bf16", aligned=False) == "two"
    wg = lambda op, dtype, n: dict(kv.split("=") for kv in rn.norm_describe(op, 64, n, dtype).split())["wg"]
    # wide chunks from 16 of them a row (2^17 vectors); 512 lanes below, and
    # always for LayerNorm with 16-bit I/O
    assert wg("rms", "bf16", N) == wg("rms_fp8", "f16", N) == wg("ln", "f32", N) == "1024"
    assert wg("rms", "f32", N // 2) == "1024" and wg("rms", "f32", N // 2 - 4) == "512"
    assert wg("rms", "bf16", N - 8) == "512" and wg("rms", "bf16", N // 4) == "512"


@pytest.mark.parametrize("dtype,M,N", [("bf16", 16, 1 << 20), ("f16", 40, 1 << 19), ("bf16", 300, 131072 + 8)])
def test_ln16_single_pass_for_few_rows_per_team(dtype, M, N):
    """LayerNorm with 16-bit I/O takes the single pass by itself when every
    team walks at most three rows (here one to three, the last shape with a
    ragged last chunk), and meets the oracle's bar."""
    import rmsnorm_forward_amd as rn
    plan = dict(kv.split("=") for kv in rn.norm_describe("ln", M, N, dtype).split())
    assert plan["mode"] == "pass" and M <= 3 * int(plan["teams"]), plan
    inp = inputs("ln", dtype, M, N, seed=M + 5)
    print(f"[gpu] LN {dtype} {M}x{N} single pass by itself: {plan['teams']} teams", flush=True)
    y, mean, rstd = run("ln", dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    compare("ln", dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what="LN 16-bit single pass")


def test_single_pass_plan():
    """On the GPU the single pass plans whole teams of resident workgroups:
    the grid is teams x chunks and holds at least one row's chunks."""
    import rmsnorm_forward_amd as rn
    import os
    os.environ["MI355NORM_PATH"] = "split1"
    try:
        d = dict(kv.split("=") for kv in rn.norm_describe("ln", 64, 1 << 20, "bf16").split())
    finally:
        del os.environ["MI355NORM_PATH"]
    assert d["mode"] == "pass" and int(d["grid"]) == int(d["teams"]) * int(d["chunks"])
    assert 1 <= int(d["teams"]) <= 64


# ---------------------------------------------------------------------------
# residual add + RMSNorm
# ---------------------------------------------------------------------------

def add_inputs(dtype, M, N, seed):
    return workloads.gen_add_rms(seed, M, N, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N", EDGE_N)
def test_add_rms_edge_shapes(dtype, N):
    M = 37 if N <= 8192 else 5
    print(f"[gpu] add_rms {dtype} M={M} N={N}", flush=True)
    inp = add_inputs(dtype, M, N, seed=N + 7)
    y, h, rstd = gpu_runner.run_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6)
    compare_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, y, h, rstd, what=f"add_rms N={N}")


@pytest.mark.parametrize("dtype,N", [("bf16", 4096), ("f32", 3000), ("bf16", 300000), ("f16", 20000)])
def test_add_rms_in_place(dtype, N):
    """y written over x and the sum over the residual give the same bits as
    separate buffers (rows, split and element-wise paths)."""
    M = 6
    print(f"[gpu] add_rms in place {dtype} M={M} N={N}", flush=True)
    inp = add_inputs(dtype, M, N, seed=N + 8)
    a = gpu_runner.run_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6)
    b = gpu_runner.run_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, inplace=True)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    compare_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, *b, what="in place")


@pytest.mark.parametrize("mode", ["split2", "splitpass"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1000, 8192, 65544, 300000])
def test_add_rms_forced_split(monkeypatch, dtype, N, mode):
    monkeypatch.setenv("MI355NORM_PATH", mode)
    M = 9
    print(f"[gpu] add_rms {mode} {dtype} M={M} N={N}", flush=True)
    inp = add_inputs(dtype, M, N, seed=N + 9)
    y, h, rstd = gpu_runner.run_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6)
    compare_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, y, h, rstd, what=f"add_rms {mode} N={N}")
    yi, hi, ri = gpu_runner.run_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, inplace=True)
    assert np.array_equal(yi.view(np.uint8), y.view(np.uint8)) and np.array_equal(hi.view(np.uint8), h.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_add_rms_unaligned_and_optional(dtype):
    M, N = 23, 4096
    inp = add_inputs(dtype, M, N, seed=31)
    y, h, rstd = gpu_runner.run_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, offset=1)
    compare_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, y, h, rstd, what="add_rms unaligned")
    y2, h2, r2 = gpu_runner.run_add(dtype, inp["x"], inp["res"], None, 1e-6, stats=False)
    compare_add(dtype, inp["x"], inp["res"], None, 1e-6, y2, h2, None, what="add_rms no gamma")
    assert r2 is None


def test_add_rms_cancellation_and_bitwise_determinism():
    """Residuals that cancel x exactly (h = 0 rows, eps > 0) and rows whose
    sums all need rounding; two calls give the same bits."""
    M, N = 8, 2048
    inp = add_inputs("bf16", M, N, seed=33)
    res = inp["res"].copy()
    res[0] = inp["x"][0] ^ np.uint16(0x8000)            # -x: the sum is exactly zero
    a = gpu_runner.run_add("bf16", inp["x"], res, inp["gamma"], 1e-6)
    b = gpu_runner.run_add("bf16", inp["x"], res, inp["gamma"], 1e-6)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    compare_add("bf16", inp["x"], res, inp["gamma"], 1e-6, *a, what="cancellation")
    assert np.all(oracle.widen(a[1][0], "bf16") == 0.0)


def test_fused_add_rms_norm_tensor_api():
    import rmsnorm_forward_amd as rn
    inp = add_inputs("bf16", 2 * 5 * 3, 1024, seed=35)
    xt = gpu_runner.to_device(inp["x"], "bf16").view(2, 5, 3, 1024)
    rt = gpu_runner.to_device(inp["res"], "bf16").view(2, 5, 3, 1024)
    gt = gpu_runner.to_device(inp["gamma"], "bf16")
    y, h, rstd = rn.fused_add_rms_norm(xt, rt, gt, eps=1e-6)
    assert y.shape == xt.shape and h.shape == xt.shape and rstd.shape == (30,)
    yh = gpu_runner.to_host(y.reshape(30, 1024), "bf16")
    hh = gpu_runner.to_host(h.reshape(30, 1024), "bf16")
    compare_add("bf16", inp["x"], inp["res"], inp["gamma"], 1e-6, yh, hh, rstd.cpu().numpy(), what="tensor api")
    y2, h2, _ = rn.fused_add_rms_norm(xt, rt, gt, eps=1e-6, inplace=True)
    assert y2.data_ptr() == xt.data_ptr() and h2.data_ptr() == rt.data_ptr()
    assert np.array_equal(gpu_runner.to_host(xt.reshape(30, 1024), "bf16"), yh)
    assert np.array_equal(gpu_runner.to_host(rt.reshape(30, 1024), "bf16"), hh)


# ---------------------------------------------------------------------------
# FP8 (E4M3) output
# ---------------------------------------------------------------------------

def compare_fp8(dtype, x, res, gamma, eps, scale, q, h, rstd, what=""):
    if res is None:
        qr, yr, rr = oracle.rms_fp8_fwd(x, gamma, dtype, eps, scale)
    else:
        hr, qr, yr, rr = oracle.add_rms_fp8_fwd(x, res, gamma, dtype, eps, scale)
        assert np.array_equal(h.view(np.uint8), hr.view(np.uint8)), f"{what}: residual sum differs"
    out = parity.check_fp8(q, qr, yr, scale, what)
    if rstd is not None:
        out.update(parity.check_stats(None, rstd, None, rr, eps, what))
    return out


@pytest.mark.parametrize("scale", [1.0, 1.0 / 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N", EDGE_N)
def test_rms_fp8_edge_shapes(dtype, N, scale):
    M = 37 if N <= 8192 else 5
    print(f"[gpu] rms_fp8 {dtype} M={M} N={N} scale={scale}", flush=True)
    inp = inputs("rms", dtype, M, N, seed=N + 11)
    q, _, rstd = gpu_runner.run_fp8(dtype, inp["x"], None, inp["gamma"], 1e-6, scale)
    compare_fp8(dtype, inp["x"], None, inp["gamma"], 1e-6, scale, q, None, rstd, what=f"rms_fp8 N={N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N", [1, 5, 1000, 4096, 8192, 16384, 65536, 131080])
def test_add_rms_fp8(dtype, N):
    M = 13 if N <= 8192 else 4
    print(f"[gpu] add_rms_fp8 {dtype} M={M} N={N}", flush=True)
    inp = add_inputs(dtype, M, N, seed=N + 12)
    q, h, rstd = gpu_runner.run_fp8(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, 0.05)
    compare_fp8(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, 0.05, q, h, rstd, what=f"add_rms_fp8 N={N}")
    qi, hi, ri = gpu_runner.run_fp8(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, 0.05, inplace=True)
    assert np.array_equal(qi, q) and np.array_equal(hi.view(np.uint8), h.view(np.uint8))


@pytest.mark.parametrize("mode", ["split2", "splitpass"])
@pytest.mark.parametrize("add", [False, True])
def test_fp8_forced_split(monkeypatch, mode, add):
    monkeypatch.setenv("MI355NORM_PATH", mode)
    M, N = 7, 300000
    inp = add_inputs("bf16", M, N, seed=14)
    res = inp["res"] if add else None
    q, h, rstd = gpu_runner.run_fp8("bf16", inp["x"], res, inp["gamma"], 1e-6, 0.02)
    compare_fp8("bf16", inp["x"], res, inp["gamma"], 1e-6, 0.02, q, h, rstd, what=f"fp8 {mode} add={add}")


def test_fp8_saturation_nan_and_unaligned():
    """A scale small enough to push many values past 448 saturates them to
    +-448; eps = 0 on an all-zero row gives NaN codes; unaligned pointers take
    the element-wise path with byte stores."""
    M, N = 9, 3000
    inp = inputs("rms", "bf16", M, N, seed=15)
    x = inp["x"].copy()
    x[3] = 0                                          # all-zero row
    q, _, rstd = gpu_runner.run_fp8("bf16", x, None, inp["gamma"], 0.0, 1e-3)
    assert np.all(np.isnan(parity.E4M3[q[3]]))
    assert np.isinf(rstd[3])
    keep = np.ones(M, bool)
    keep[3] = False
    vals = parity.E4M3[q[keep]]
    assert np.mean(np.abs(vals) == 448.0) > 0.3          # |y| > 0.448 saturates: about 40%
    compare_fp8("bf16", x[keep], None, inp["gamma"], 0.0, 1e-3, q[keep], None, rstd[keep], what="saturated")
    q2, _, r2 = gpu_runner.run_fp8("bf16", inp["x"], None, inp["gamma"], 1e-6, 0.1, offset=1)
    compare_fp8("bf16", inp["x"], None, inp["gamma"], 1e-6, 0.1, q2, None, r2, what="fp8 unaligned")


def test_fp8_tensor_api():
    import rmsnorm_forward_amd as rn
    inp = add_inputs("bf16", 24, 2048, seed=16)
    xt = gpu_runner.to_device(inp["x"], "bf16").view(4, 6, 2048)
    rt = gpu_runner.to_device(inp["res"], "bf16").view(4, 6, 2048)
    gt = gpu_runner.to_device(inp["gamma"], "bf16")
    q, rstd = rn.rms_norm_fp8(xt, gt, scale=0.03, eps=1e-6)
    assert q.dtype == torch.float8_e4m3fn and q.shape == xt.shape
    compare_fp8("bf16", inp["x"], None, inp["gamma"], 1e-6, 0.03, q.view(torch.uint8).reshape(24, 2048).cpu().numpy(),
                None, rstd.cpu().numpy(), what="fp8 tensor api")
    q, h, rstd = rn.fused_add_rms_norm_fp8(xt, rt, gt, scale=0.03, eps=1e-6)
    compare_fp8("bf16", inp["x"], inp["res"], inp["gamma"], 1e-6, 0.03,
                q.view(torch.uint8).reshape(24, 2048).cpu().numpy(),
                gpu_runner.to_host(h.reshape(24, 2048), "bf16"), rstd.cpu().numpy(), what="fp8 add tensor api")


# ---------------------------------------------------------------------------
# row strides (norm_fwd)
# ---------------------------------------------------------------------------

STRIDE_CASES = [
    # (dtype, N, ldx, ldy, offset): vector path, element-wise path (row
    # starts off 16 bytes), long rows on the split path, odd widths
    ("bf16", 4096, 4096 + 64, 4096 + 8, 0),
    ("bf16", 4096, 4096 + 3, 4096 + 8, 0),
    ("f32", 1000, 1024, 1000, 4),
    ("f16", 2056, 2056 + 8, 2056 + 16, 8),
    ("bf16", 140000, 140000 + 8, 140008, 0),
    ("f32", 70000, 70004, 70000 + 36, 0),
    # rows of 2^17 16-byte vectors: the single pass's wide chunks
    ("bf16", 1 << 20, (1 << 20) + 64, (1 << 20) + 8, 0),
    ("f32", 1 << 19, (1 << 19) + 4, (1 << 19) + 12, 0),
]


@pytest.mark.parametrize("op", ["ln", "rms", "add_rms", "rms_fp8", "add_rms_fp8"])
@pytest.mark.parametrize("dtype,N,ldx,ldy,offset", STRIDE_CASES)
def test_strided_rows(op, dtype, N, ldx, ldy, offset):
    """Rows ld elements apart (no copy) give the contiguous results, and no
    byte between the rows of an output is written."""
    M = 5
    print(f"[gpu] strided {op} {dtype} N={N} ldx={ldx} ldy={ldy} offset={offset}", flush=True)
    add = op.startswith("add")
    inp = add_inputs(dtype, M, N, seed=N + 21) if add else inputs("rms" if "rms" in op else "ln", dtype, M, N,
                                                                   seed=N + 21)
    scale = 0.05
    beta = inp["beta"] if op == "ln" else None
    y, h, mean, rstd = gpu_runner.run_strided(op, dtype, inp["x"], inp["gamma"], beta, 1e-5,
                                              res=inp.get("res"), scale=scale, ldx=ldx, ldy=ldy,
                                              ldr=ldx + 8, ldh=ldy + 24, offset=offset)
    if op == "ln":
        compare("ln", dtype, inp["x"], inp["gamma"], beta, 1e-5, y, mean, rstd, what="strided ln")
    elif op == "rms":
        compare("rms", dtype, inp["x"], inp["gamma"], None, 1e-5, y, None, rstd, what="strided rms")
    elif op == "add_rms":
        compare_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-5, y, h, rstd, what="strided add_rms")
    else:
        compare_fp8(dtype, inp["x"], inp.get("res"), inp["gamma"], 1e-5, scale, y, h, rstd,
                    what=f"strided {op}")


# x alone off a 16-byte boundary (a view into a larger buffer), everything
# else aligned: the kernels read x in aligned 16-byte blocks and realign them
# in registers.  (dtype, N, M): row tiles of 8 to 1024 lanes, several rows
# per wavefront with ragged vector rows (f16 1000, bf16 8 and 24), one
# wavefront per row (bf16 2048 and 5120), 16 vectors per lane (RMSNorm fp32
# 2048);
# split rows on the two kernels, with a ragged last chunk (bf16 140000, fp32
# 70000) and without (f16 2^20).
REALIGN_CASES = [("bf16", 4096, 6), ("f16", 1000, 37), ("bf16", 8, 70), ("bf16", 24, 41), ("f32", 8192, 5),
                 ("bf16", 2048, 9),
                 ("bf16", 5120, 4), ("bf16", 65536, 3), ("f32", 2048, 9), ("f16", 256, 19),
                 ("bf16", 140000, 3), ("f32", 70000, 3), ("f16", 1 << 20, 2)]


@pytest.mark.parametrize("op", ["ln", "rms", "rms_fp8"])
@pytest.mark.parametrize("dtype,N,M", REALIGN_CASES)
def test_realigned_x(monkeypatch, op, dtype, N, M):
    """Misaligned x by every element offset within 16 bytes, with row strides
    that keep or change the offset from row to row: the same bits as the same
    call, on the same tile, on an aligned contiguous copy of x (the arithmetic
    is the same), and the oracle's results."""
    import rmsnorm_forward_amd as rn
    plan = rn.norm_describe(op, M, N, dtype, aligned="x")
    assert "x=realigned" in plan, plan
    f = dict(kv.split("=") for kv in plan.split())
    if f["path"] == "rows":
        monkeypatch.setenv("MI355NORM_TILE", f"{f['team']}x{f['vpl']}")
    else:
        assert f["mode"] == "two", plan
        monkeypatch.setenv("MI355NORM_PATH", "split2")
    epv = 16 // {"f32": 4, "bf16": 2, "f16": 2}[dtype]
    inp = inputs("rms" if "rms" in op else "ln", dtype, M, N, seed=N + 31)
    beta = inp["beta"] if op == "ln" else None
    scale = 0.05
    ref = gpu_runner.run_strided(op, dtype, inp["x"], inp["gamma"], beta, 1e-5, scale=scale, ldx=N, ldy=N)
    for k in range(1, epv):
        for ldx in (N, N + 1, N + epv - 1, N + 3 * epv):
            print(f"[gpu] realigned x {op} {dtype} M={M} N={N} x_offset={k} ldx={ldx}", flush=True)
            got = gpu_runner.run_strided(op, dtype, inp["x"], inp["gamma"], beta, 1e-5, scale=scale, ldx=ldx,
                                         ldy=N, x_offset=k)
            for name, a, b in zip(("y", "h", "mean", "rstd"), got, ref):
                if a is None:
                    continue
                assert a.tobytes() == b.tobytes(), f"{name} differs from the aligned call (x_offset={k}, ldx={ldx})"
    if op == "rms_fp8":
        compare_fp8(dtype, inp["x"], None, inp["gamma"], 1e-5, scale, got[0], None, got[3], what="realigned fp8")
    else:
        compare(op, dtype, inp["x"], inp["gamma"], beta, 1e-5, got[0], got[2], got[3], what=f"realigned {op}")


@pytest.mark.parametrize("N", [2048, 140000])
def test_strided_in_place_and_interleaved(N):
    """The fused residual add in place on strided rows; and LayerNorm of the
    left half of a [M, 2N] buffer into its right half."""
    M, dtype = 4, "bf16"
    inp = add_inputs(dtype, M, N, seed=N + 22)
    a = gpu_runner.run_strided("add_rms", dtype, inp["x"], inp["gamma"], None, 1e-6, res=inp["res"],
                               ldx=N + 64, ldy=N + 64, ldr=N + 32, inplace=True)
    compare_add(dtype, inp["x"], inp["res"], inp["gamma"], 1e-6, a[0], a[1], a[3], what="strided in place")
    # interleaved: x in columns [0, N), y in [N, 2N) of one buffer
    import rmsnorm_forward_amd as rn
    li = inputs("ln", dtype, M, N, seed=N + 23)
    buf = torch.zeros(M, 2 * N, dtype=torch.bfloat16, device="cuda")
    buf[:, :N] = gpu_runner.to_device(li["x"], dtype).view(M, N)
    gt, bt = gpu_runner.to_device(li["gamma"], dtype), gpu_runner.to_device(li["beta"], dtype)
    mean = torch.empty(M, device="cuda")
    rstd = torch.empty(M, device="cuda")
    st = rn.norm_fwd("ln", dtype, M, N, buf.data_ptr(), buf[:, N:].data_ptr(), ld_x=2 * N, ld_y=2 * N,
                     gamma=gt.data_ptr(), beta=bt.data_ptr(), mean=mean.data_ptr(), rstd=rstd.data_ptr(),
                     eps=1e-5, stream=torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_OK
    torch.cuda.synchronize()
    y = gpu_runner.to_host(buf[:, N:].contiguous().view(-1), dtype).reshape(M, N)
    x_after = gpu_runner.to_host(buf[:, :N].contiguous().view(-1), dtype).reshape(M, N)
    assert np.array_equal(x_after, li["x"])
    compare("ln", dtype, li["x"], li["gamma"], li["beta"], 1e-5, y, mean.cpu().numpy(), rstd.cpu().numpy(),
            what="interleaved")


def test_tensor_api_takes_strided_rows_without_copy():
    import rmsnorm_forward_amd as rn
    M, N = 6, 1024
    li = inputs("ln", "bf16", M, N, seed=24)
    big = torch.zeros(M, N + 128, dtype=torch.bfloat16, device="cuda")
    big[:, 64:64 + N] = gpu_runner.to_device(li["x"], "bf16").view(M, N)
    xv = big[:, 64:64 + N]                          # strided view, not contiguous
    assert not xv.is_contiguous()
    y, mean, rstd = rn.layer_norm(xv, gpu_runner.to_device(li["gamma"], "bf16"),
                                  gpu_runner.to_device(li["beta"], "bf16"), eps=1e-5)
    compare("ln", "bf16", li["x"], li["gamma"], li["beta"], 1e-5,
            gpu_runner.to_host(y.reshape(-1), "bf16").reshape(M, N), mean.cpu().numpy(), rstd.cpu().numpy(),
            what="tensor api strided")


def test_m_zero_launches_nothing():
    import rmsnorm_forward_amd as rn
    st = rn.ln_fwd(None, None, None, None, None, None, 0, 128, 1e-5, rn.NORM_BF16,
                   torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_OK


def test_tensor_api_matches_abi():
    import rmsnorm_forward_amd as rn
    inp = inputs("ln", "bf16", 2 * 3 * 7, 768, seed=51)
    xt = gpu_runner.to_device(inp["x"], "bf16").view(2, 3, 7, 768)
    gt = gpu_runner.to_device(inp["gamma"], "bf16")
    bt = gpu_runner.to_device(inp["beta"], "bf16")
    y, mean, rstd = rn.layer_norm(xt, gt, bt, eps=1e-5)
    torch.cuda.synchronize()
    assert y.shape == (2, 3, 7, 768) and mean.dtype == torch.float32 and mean.shape == (42,)
    y2, m2, r2 = run("ln", "bf16", inp["x"], inp["gamma"], inp["beta"], 1e-5)
    assert np.array_equal(gpu_runner.to_host(y.reshape(42, 768), "bf16"), y2)
    yr, rr = rn.rms_norm(xt, gt, eps=1e-6)
    torch.cuda.synchronize()
    y3, _, r3 = run("rms", "bf16", inp["x"], inp["gamma"], None, 1e-6)
    assert np.array_equal(gpu_runner.to_host(yr.reshape(42, 768), "bf16"), y3)


@pytest.mark.parametrize("op,dtype,offset", [("ln", "f32", 0), ("rms", "bf16", 1)])
def test_maximum_row_length(op, dtype, offset):
    """N = 2^24, the largest row the ABI takes, on the split path (aligned
    and element-wise)."""
    M, N = 2, 1 << 24
    print(f"[gpu] maximum N {op} {dtype} offset={offset}", flush=True)
    inp = inputs(op, dtype, M, N, seed=24)
    y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, offset=offset)
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what="N = 2^24")


@pytest.mark.parametrize("dtype,N", [("bf16", 1000), ("f32", 8192), ("bf16", 24)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_grid_stride_over_row_groups(monkeypatch, op, dtype, N):
    """A grid far smaller than the row groups (each workgroup walks many):
    the same bits as the one-group-per-workgroup launch, and the oracle's
    values."""
    M = 1001
    inp = inputs(op, dtype, M, N, seed=N + 31)
    y0, m0, r0 = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    monkeypatch.setenv("MI355NORM_GRID", "7")
    print(f"[gpu] grid 7 {op} {dtype} M={M} N={N}", flush=True)
    y, mean, rstd = run(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5)
    assert np.array_equal(y.view(np.uint8), y0.view(np.uint8)) and np.array_equal(rstd, r0)
    compare(op, dtype, inp["x"], inp["gamma"], inp["beta"], 1e-5, y, mean, rstd, what="grid 7")
