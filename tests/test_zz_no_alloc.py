"""norm_fwd_noalloc, the forward entry point that allocates nothing, against
norm_fwd (the entry point it is a variant of) through the C ABI.

Rows too long for one workgroup keep their partial statistics in the
library's fixed device scratch instead of an allocated workspace; the kernels
are the same, so the results must be the same bits.  Two calls in a row, the
second smaller (the scratch keeps the first call's contents), then a row-path
call; then the refusals: a call needing more scratch than the fixed array
holds, and the single-pass schedule."""
from __future__ import annotations

import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
gpu_runner = pytest.importorskip("gpu_runner")
rn = pytest.importorskip("rmsnorm_forward_amd")

# (op, dtype, M, N, element offset of every buffer: 1 = unaligned, element-wise path)
CALLS = [
    ("ln", "bf16", 6, 1 << 18, 0),        # split rows, 16-byte vectors, 16 chunks per row
    ("rms", "f32", 3, 100003, 1),         # smaller, split rows, element-wise
    ("add_rms", "bf16", 2, 70000, 0),     # residual add on split rows, 16-byte vectors
    ("ln", "bf16", 37, 4096, 0),          # row kernel: no scratch
]


def _inputs(op, dtype, M, N, seed):
    if op == "ln":
        return workloads.gen_ln_normal(seed, M, N, dtype, loc=3.0, scale=2.0)
    if op == "add_rms":
        return workloads.gen_add_rms(seed, M, N, dtype)
    return workloads.gen_rms_uniform(seed, M, N, dtype)


def _call(fn, op, dtype, M, N, off, inp, x_off=None):
    dev = lambda a: gpu_runner.to_device(a, dtype, off) if a is not None else None
    x = gpu_runner.to_device(inp["x"], dtype, off if x_off is None else x_off)
    g = dev(inp["gamma"])
    b = dev(inp.get("beta")) if op == "ln" else None
    res = dev(inp["res"]) if op == "add_rms" else None
    tdt = gpu_runner.TORCH_DT[dtype]
    y = torch.full((M * N + off,), float("nan"), dtype=tdt, device="cuda")[off:]
    h = torch.zeros(M * N + off, dtype=tdt, device="cuda")[off:] if op == "add_rms" else None
    mean = torch.full((M,), float("nan"), device="cuda") if op == "ln" else None
    rstd = torch.full((M,), float("nan"), device="cuda")
    p = lambda t: t.data_ptr() if t is not None else None
    eps = 1e-5 if op == "ln" else 1e-6
    print(f"[gpu] {fn.__name__} {op} {dtype} {M}x{N} offset {off} x offset {x_off}", flush=True)
    st = fn(op, dtype, M, N, p(x), p(y), residual=p(res), gamma=p(g), beta=p(b), residual_out=p(h),
            mean=p(mean), rstd=p(rstd), eps=eps, stream=torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_OK, f"{rn.STATUS.get(st)}: {rn.norm_status_str(st)} [{rn.norm_last_error()}]"
    torch.cuda.synchronize()
    out = [gpu_runner.to_host(y, dtype), rstd.cpu().numpy()]
    if mean is not None:
        out.append(mean.cpu().numpy())
    if h is not None:
        out.append(gpu_runner.to_host(h, dtype))
    return out


def test_noalloc_gives_norm_fwd_bits_on_consecutive_calls():
    for k, (op, dtype, M, N, off) in enumerate(CALLS):
        plan = rn.norm_describe(op, M, N, dtype, aligned=(off == 0 and (N * (4 if dtype == "f32" else 2)) % 16 == 0))
        assert ("path=split" in plan) == (N > 16384), plan
        inp = _inputs(op, dtype, M, N, 900 + k)
        got = _call(rn.norm_fwd_noalloc, op, dtype, M, N, off, inp)
        want = _call(rn.norm_fwd, op, dtype, M, N, off, inp)
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"call {k} ({op} {dtype} {M}x{N}) differs"
        assert np.all(np.isfinite(got[1]))


def test_noalloc_realigned_x_gives_norm_fwd_bits():
    """x alone off 16 bytes: both entry points take the realigned kernels
    (split rows: the two kernels, partials in the fixed scratch for
    norm_fwd_noalloc), so the bits are the same; consecutive calls, each
    smaller than the one before."""
    for k, (op, dtype, M, N, x_off) in enumerate([("rms", "bf16", 4, 1 << 18, 3), ("ln", "f32", 3, 70000, 1),
                                                  ("ln", "bf16", 9, 4096, 5)]):
        plan = dict(kv.split("=") for kv in rn.norm_describe(op, M, N, dtype, aligned="x").split())
        assert plan["x"] == "realigned" and plan.get("mode", "two") == "two", plan
        inp = _inputs(op, dtype, M, N, 970 + k)
        got = _call(rn.norm_fwd_noalloc, op, dtype, M, N, 0, inp, x_off=x_off)
        want = _call(rn.norm_fwd, op, dtype, M, N, 0, inp, x_off=x_off)
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"call {k} ({op} {dtype} {M}x{N}) differs"
        assert np.all(np.isfinite(got[1]))


def test_noalloc_takes_the_two_kernels_where_norm_fwd_takes_the_single_pass():
    """RMSNorm rows split across workgroups: norm_fwd's automatic choice is
    the single pass, whose per-row slots live in the allocated workspace;
    norm_fwd_noalloc then runs the two-kernel form on its fixed scratch.  The
    two chunk a row differently, so the bits may differ: each is compared
    with the oracle at the parity bar (fp32 y within 2e-5, rstd within 1e-5
    relative; bf16 y within one ulp)."""
    import parity
    import oracle
    for k, (dtype, M, N) in enumerate([("f32", 4, 100000), ("bf16", 3, 1 << 18)]):
        plan = dict(kv.split("=") for kv in rn.norm_describe("rms", M, N, dtype).split())
        assert plan["path"] == "split" and plan["mode"] == "pass", plan
        inp = _inputs("rms", dtype, M, N, 950 + k)
        yr, rr = oracle.rms_fwd(inp["x"], inp["gamma"], dtype, 1e-6)
        for fn in (rn.norm_fwd_noalloc, rn.norm_fwd):
            y, rstd = _call(fn, "rms", dtype, M, N, 0, inp)
            parity.check_y(y.reshape(M, N), yr, dtype, f"{fn.__name__} rms {dtype} {M}x{N}")
            parity.check_stats(None, rstd, None, rr, 1e-6, f"{fn.__name__} rms {dtype} {M}x{N}")


def test_noalloc_refuses_what_its_scratch_cannot_hold(monkeypatch):
    M, N = 40, 100000
    x = torch.zeros(M * N, dtype=torch.float32, device="cuda")
    y = torch.full((M * N,), 7.0, device="cuda")
    # rows so short that a forced split batches 2^20 of them: 8 MiB of partials
    monkeypatch.setenv("MI355NORM_PATH", "split")
    Ms, Ns = 1 << 20, 64
    xs = torch.zeros(Ms * Ns, dtype=torch.float32, device="cuda")
    ys = torch.full((Ms * Ns,), 7.0, device="cuda")
    st = rn.norm_fwd_noalloc("rms", "f32", Ms, Ns, xs.data_ptr(), ys.data_ptr(), eps=1e-6,
                             stream=torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_ERR_SCRATCH, rn.STATUS.get(st)
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    st = rn.norm_fwd_noalloc("rms", "f32", M, N, x.data_ptr(), y.data_ptr(), eps=1e-6,
                             stream=torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_ERR_BAD_ARG, rn.STATUS.get(st)
    torch.cuda.synchronize()
    assert bool((ys == 7.0).all()) and bool((y == 7.0).all()), "a refused call wrote its output"
