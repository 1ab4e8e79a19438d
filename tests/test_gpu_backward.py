"""LayerNorm / RMSNorm backward (ln_bwd, rms_bwd) on the GPU vs the CPU
oracle, through the C ABI, at the bound derived in tests/parity.py.

Both sides get the same fp32 statistics: the oracle's forward mean / rstd
rounded to fp32 (what a forward pass stores).  Shapes: the measured
backward configurations at full size, every row length class of the row
kernel (up to 32768; longer rows are in test_gpu_backward_split.py) with
ragged row counts, unaligned pointers, in-place dx, the
optional gamma / dgamma / dbeta, M = 0, every tile, forced grids, and bitwise
determinism, and the large-mean stress rows of the forward.
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
rn = pytest.importorskip("rmsnorm_forward_amd")

EPS = {"ln": 1e-5, "rms": 1e-6}
E = {"f32": 4, "f16": 2, "bf16": 2}


def inputs(op, dtype, M, N, seed):
    d = workloads.gen_bwd(seed, M, N, dtype, op + "_bwd")
    if op == "ln":
        _, mean, rstd = oracle.ln_fwd(d["x"], d["gamma"], None, dtype, EPS[op])
        mean = mean.astype(np.float32)
    else:
        _, rstd = oracle.rms_fwd(d["x"], d["gamma"], dtype, EPS[op])
        mean = None
    return d["dy"], d["x"], d["gamma"], mean, rstd.astype(np.float32)


def plan(op, M, N, dtype, aligned=True):
    d = dict(kv.split("=") for kv in rn.norm_bwd_describe(op, M, N, dtype, aligned).split())
    return {k: (v if k in ("path", "op", "mode") else int(v)) for k, v in d.items()}


def go(op, dtype, M, N, seed=0, offset=0, **kw):
    dy, x, g, mean, rstd = inputs(op, dtype, M, N, seed)
    print(f"[bwd] {op} {dtype} M={M} N={N} offset={offset} {kw}", flush=True)
    dx, dg, db = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd, offset=offset, **kw)
    aligned = offset == 0 and (N * E[dtype]) % 16 == 0
    st = parity.check_bwd(op, dtype, dy, x, g, mean, rstd, dx, dg, db, plan(op, M, N, dtype, aligned),
                          what=f"{op} {dtype} {M}x{N}")
    return st, (dx, dg, db)


@pytest.mark.parametrize("name", [n for n, w in workloads.CONFIGS.items() if w.op.endswith("_bwd")])
def test_measured_backward_configuration(name):
    w = workloads.CONFIGS[name]
    op = w.op[:-4]
    d = workloads.generate(name)
    if op == "ln":
        _, mean, rstd = oracle.ln_fwd(d["x"], d["gamma"], None, w.dtype, w.eps)
        mean = mean.astype(np.float32)
    else:
        _, rstd = oracle.rms_fwd(d["x"], d["gamma"], w.dtype, w.eps)
        mean = None
    rstd = rstd.astype(np.float32)
    print(f"[bwd] {name}", flush=True)
    dx, dg, db = gpu_runner.run_bwd(op, w.dtype, d["dy"], d["x"], d["gamma"], mean, rstd)
    st = parity.check_bwd(op, w.dtype, d["dy"], d["x"], d["gamma"], mean, rstd, dx, dg, db,
                          plan(op, w.M, w.N, w.dtype), what=name)
    print(name, st)


BWD_N = [1, 7, 8, 64, 100, 768, 1000, 1024, 2056, 4096, 5120, 8192, 12288, 16384, 24576, 32768]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["ln", "rms"])
@pytest.mark.parametrize("N", BWD_N)
def test_backward_row_lengths(op, dtype, N):
    M = 300 if N <= 4096 else 40
    go(op, dtype, M, N, seed=N)


@pytest.mark.parametrize("M", [1, 2, 37, 513, 5000])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_backward_ragged_row_counts(op, M):
    # more row groups than workgroups (rows grid-strided), fewer, and one
    go(op, "bf16", M, 1000, seed=M)
    go(op, "f32", M, 256, seed=M + 1)


@pytest.mark.parametrize("dtype,N", [("f32", 4096), ("bf16", 16384), ("f16", 1000), ("bf16", 64)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_backward_unaligned_pointers(op, dtype, N):
    go(op, dtype, 64, N, seed=7, offset=1)


@pytest.mark.parametrize("which", ["dy", "x"])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_backward_in_place(op, which):
    ref, (dx0, dg0, db0) = go(op, "bf16", 200, 4096, seed=3)
    _, (dx1, dg1, db1) = go(op, "bf16", 200, 4096, seed=3, inplace=which)
    assert np.array_equal(dx0, dx1) and np.array_equal(dg0, dg1)


@pytest.mark.parametrize("op", ["ln", "rms"])
def test_backward_optional_outputs_and_gamma(op):
    dy, x, g, mean, rstd = inputs(op, "f32", 100, 768, 11)
    for gamma, want_g, want_b in [(None, True, True), (g, False, True), (g, True, False), (g, False, False)]:
        dx, dg, db = gpu_runner.run_bwd(op, "f32", dy, x, gamma, mean, rstd, want_g=want_g, want_b=want_b)
        parity.check_bwd(op, "f32", dy, x, gamma, mean, rstd, dx, dg, db, plan(op, 100, 768, "f32"),
                         what=f"gamma={gamma is not None} dg={want_g} db={want_b}")
        assert (dg is None) == (not want_g)


def test_backward_no_rows_gives_zero_sums():
    N = 1000
    dg = torch.full((N,), float("nan"), device="cuda")
    db = torch.full((N,), float("nan"), device="cuda")
    st = rn.ln_bwd(None, None, None, None, None, None, dg.data_ptr(), db.data_ptr(), 0, N, rn.NORM_F32,
                   torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_OK
    assert torch.all(dg == 0) and torch.all(db == 0)


@pytest.mark.parametrize("dtype,N", [("bf16", 4096), ("f32", 1000)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_backward_every_tile(monkeypatch, op, dtype, N):
    dy, x, g, mean, rstd = inputs(op, dtype, 70, N, 5)
    epv = 16 // E[dtype] if (N * E[dtype]) % 16 == 0 else 1
    nv = N // epv
    ran = 0
    for team in (8, 16, 32, 64, 128, 256, 512, 1024):
        for vpl in (1, 2, 4, 8, 16):
            if team * vpl < nv or vpl * epv > 32:
                continue
            monkeypatch.setenv("MI355NORM_TILE", f"{team}x{vpl}")
            p = plan(op, 70, N, dtype)
            print(f"[bwd] tile {team}x{vpl}", flush=True)
            dx, dg, db = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd)
            parity.check_bwd(op, dtype, dy, x, g, mean, rstd, dx, dg, db, p, what=f"tile {team}x{vpl}")
            ran += 1
    assert ran >= 3


@pytest.mark.parametrize("grid", [1, 3, 1000])
def test_backward_forced_grid(monkeypatch, grid):
    monkeypatch.setenv("MI355NORM_GRID", str(grid))
    for op in ("ln", "rms"):
        go(op, "bf16", 777, 2048, seed=grid)


def test_backward_is_bitwise_deterministic():
    dy, x, g, mean, rstd = inputs("ln", "bf16", 3000, 4096, 21)
    a = gpu_runner.run_bwd("ln", "bf16", dy, x, g, mean, rstd)
    b = gpu_runner.run_bwd("ln", "bf16", dy, x, g, mean, rstd)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_backward_workspace_shared_with_forward_split():
    # the split forward and the backward share the stream's workspace
    go("rms", "bf16", 600, 8192, seed=31)
    xs = workloads.gen_ln_normal(5, 4, 300000, "bf16")
    y, m, r = gpu_runner.run("ln", "bf16", xs["x"], xs["gamma"], xs["beta"], 1e-5)
    yr, mr, rr = oracle.ln_fwd(xs["x"], xs["gamma"], xs["beta"], "bf16", 1e-5)
    parity.check_y(y, yr, "bf16", "split after backward")
    go("ln", "bf16", 5000, 8192, seed=32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_autograd_functions(dtype):
    """layer_norm_autograd / rms_norm_autograd: gradients equal the direct
    backward calls bit for bit, and agree with the oracle's backward given
    the oracle's own statistics to within the forward's statistics error."""
    tdt = gpu_runner.TORCH_DT[dtype]
    M, N = 64, 1024
    for op in ("ln", "rms"):
        dy, x, g, mean, rstd = inputs(op, dtype, M, N, 41)
        xt = gpu_runner.to_device(x, dtype).view(M, N).clone().requires_grad_(True)
        gt = gpu_runner.to_device(g, dtype).clone().requires_grad_(True)
        dyt = gpu_runner.to_device(dy, dtype).view(M, N)
        if op == "ln":
            bt = torch.zeros(N, dtype=tdt, device="cuda", requires_grad=True)
            y = rn.layer_norm_autograd(xt, gt, bt, EPS[op])
            y.backward(dyt)
            _, m2, r2 = rn.layer_norm(xt.detach(), gt.detach(), bt.detach(), EPS[op])
            dx, dg, db = rn.layer_norm_backward(dyt, xt.detach(), m2, r2, gt.detach())
            assert torch.equal(bt.grad, db.to(tdt))
        else:
            y = rn.rms_norm_autograd(xt, gt, EPS[op])
            y.backward(dyt)
            _, r2 = rn.rms_norm(xt.detach(), gt.detach(), EPS[op])
            dx, dg = rn.rms_norm_backward(dyt, xt.detach(), r2, gt.detach())
        assert torch.equal(xt.grad, dx) and torch.equal(gt.grad, dg.to(tdt))
        # against the oracle: the forward's statistics differ from the
        # oracle's by <= 1e-5 relative, so the bound is loosened to 1e-4 of
        # each row's gradient scale
        ref = (oracle.ln_bwd(dy, x, g, dtype, mean, rstd) if op == "ln" else
               oracle.rms_bwd(dy, x, g, dtype, rstd))
        got = gpu_runner.to_host(xt.grad, dtype).reshape(M, N)
        got = got.astype(np.float64) if dtype == "f32" else oracle.widen(got, dtype)
        scale = np.abs(ref[0]).max(1, keepdims=True)
        tol = 1e-4 * scale + (0 if dtype == "f32" else parity.ulp_of(np.abs(ref[0]) + 1e-4 * scale, dtype))
        assert np.all(np.abs(got - ref[0]) <= tol), op


@pytest.mark.parametrize("dtype,N,lddy,ldx,lddx,offset", [
    ("bf16", 4096, 4096 + 64, 4096 + 8, 4096 + 128, 0),      # 16-byte aligned rows
    ("bf16", 4096, 4096 + 3, 4096, 4096 + 5, 0),             # unaligned strides: element-wise path
    ("f32", 1000, 1000 + 4, 1000 + 12, 1000 + 36, 0),
    ("f16", 7, 16, 24, 8, 1),
    ("bf16", 16384, 16384 + 64, 16384 + 64, 16384 + 8, 0),
])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_backward_strided_rows(op, dtype, N, lddy, ldx, lddx, offset):
    M = 9
    dy, x, g, mean, rstd = inputs(op, dtype, M, N, N + 61)
    print(f"[bwd] strided {op} {dtype} N={N} ld={lddy},{ldx},{lddx} offset={offset}", flush=True)
    dx, dg, db = gpu_runner.run_bwd_strided(op, dtype, dy, x, g, mean, rstd, lddy=lddy, ldx=ldx, lddx=lddx,
                                            offset=offset)
    aligned = offset == 0 and all((v * E[dtype]) % 16 == 0 for v in (N, lddy, ldx, lddx))
    parity.check_bwd(op, dtype, dy, x, g, mean, rstd, dx, dg, db, plan(op, M, N, dtype, aligned),
                     what=f"strided {op}")


@pytest.mark.parametrize("which", ["dy", "x"])
def test_backward_strided_in_place(which):
    M, N = 6, 2048
    dy, x, g, mean, rstd = inputs("ln", "bf16", M, N, 71)
    dx, dg, db = gpu_runner.run_bwd_strided("ln", "bf16", dy, x, g, mean, rstd, lddy=N + 64, ldx=N + 128,
                                            lddx=0, inplace=which)
    parity.check_bwd("ln", "bf16", dy, x, g, mean, rstd, dx, dg, db, plan("ln", M, N, "bf16"), what="in place")


def test_backward_tensor_api_takes_strided_rows():
    """layer_norm_backward / rms_norm_backward on column slices of wider
    tensors give the same bits as on contiguous copies."""
    M, N = 8, 1024
    for op in ("ln", "rms"):
        dy, x, g, mean, rstd = inputs(op, "bf16", M, N, 81)
        wide_x = torch.zeros(M, 2 * N, dtype=torch.bfloat16, device="cuda")
        wide_dy = torch.zeros(M, 3 * N, dtype=torch.bfloat16, device="cuda")
        wide_x[:, N:] = gpu_runner.to_device(x, "bf16").view(M, N)
        wide_dy[:, :N] = gpu_runner.to_device(dy, "bf16").view(M, N)
        xs, dys = wide_x[:, N:], wide_dy[:, :N]
        assert not xs.is_contiguous() and not dys.is_contiguous()
        gt = gpu_runner.to_device(g, "bf16")
        rt = torch.from_numpy(rstd).cuda()
        if op == "ln":
            mt = torch.from_numpy(mean).cuda()
            a = rn.layer_norm_backward(dys, xs, mt, rt, gt)
            b = rn.layer_norm_backward(dys.contiguous(), xs.contiguous(), mt, rt, gt)
        else:
            a = rn.rms_norm_backward(dys, xs, rt, gt) + (None,)
            b = rn.rms_norm_backward(dys.contiguous(), xs.contiguous(), rt, gt) + (None,)
        for u, v in zip(a, b):
            assert (u is None and v is None) or torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                                                            v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_on_large_mean_stress_rows(dtype):
    """The forward's stress recipe (rows of 1000 + N(0, 1e-2), outlier
    channels x100) under the LayerNorm backward: x - mean cancels almost
    completely on the large-mean rows, and both sides take the same fp32
    statistics; dx, dgamma and dbeta meet the bound and stay finite."""
    M, N = 512, 8192
    s = workloads.gen_ln_stress(1012, M, N, dtype)
    rng = np.random.default_rng(1013)
    dy = workloads.to_storage(rng.standard_normal((M, N)), dtype)
    _, mean, rstd = oracle.ln_fwd(s["x"], s["gamma"], None, dtype, 1e-5)
    mean, rstd = mean.astype(np.float32), rstd.astype(np.float32)
    print(f"[bwd] stress {dtype}", flush=True)
    dx, dg, db = gpu_runner.run_bwd("ln", dtype, dy, s["x"], s["gamma"], mean, rstd)
    parity.check_bwd("ln", dtype, dy, s["x"], s["gamma"], mean, rstd, dx, dg, db, plan("ln", M, N, dtype),
                     what=f"stress {dtype}")
    got = dx.astype(np.float64) if dtype == "f32" else oracle.widen(dx, dtype)
    assert np.isfinite(got).all() and np.isfinite(dg).all() and np.isfinite(db).all()
