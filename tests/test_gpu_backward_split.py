"""The split-row backward (rows longer than one workgroup's tile, up to
N = 2^24, or any row with MI355NORM_PATH=split) on the GPU vs the CPU
oracle, through the C ABI, at the bound derived in tests/parity.py.

Shapes: long rows of each dtype (aligned and element-wise), the largest row
the ABI takes, short rows forced onto the split path (ragged chunk tails),
several batches of rows with a short last batch (the accumulating partial
rows), a sums grid far smaller than its work items, unaligned pointers,
strided rows, in-place dx, the optional gamma / dgamma / dbeta, M = 0, and
bitwise determinism; the single pass (forced, and where the planner takes
it by itself) on long and
short rows, in place, deterministic, and with its bounded wait forced to
time out from the host.
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
gpu_runner = pytest.importorskip("gpu_runner")
rn = pytest.importorskip("rmsnorm_forward_amd")

from test_gpu_backward import E, inputs, plan  # noqa: E402


def go(op, dtype, M, N, seed=0, offset=0, **kw):
    dy, x, g, mean, rstd = inputs(op, dtype, M, N, seed)
    aligned = offset == 0 and (N * E[dtype]) % 16 == 0
    p = plan(op, M, N, dtype, aligned)
    assert p["path"] == "bwd_split", p
    print(f"[bwd split] {op} {dtype} M={M} N={N} offset={offset} {kw} {p}", flush=True)
    dx, dg, db = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd, offset=offset, **kw)
    st = parity.check_bwd(op, dtype, dy, x, g, mean, rstd, dx, dg, db, p, what=f"split {op} {dtype} {M}x{N}")
    return st, (dx, dg, db)


@pytest.mark.parametrize("dtype,N", [("bf16", 32776), ("f32", 40000), ("f16", 65544), ("bf16", 100000),
                                     ("f32", 1 << 20), ("f16", 16385), ("bf16", 30001)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_backward_long_rows(op, dtype, N):
    """Rows past the row kernel's limit (32768 elements; 16384 when the rows
    are not 16-byte aligned) take the split path by themselves."""
    M = 4 if N > 100000 else 24
    go(op, dtype, M, N, seed=N)


@pytest.mark.parametrize("op,dtype,offset", [("ln", "f32", 0), ("rms", "bf16", 1)])
def test_split_backward_maximum_row_length(op, dtype, offset):
    """N = 2^24, the largest row the ABI takes (aligned and element-wise)."""
    go(op, dtype, 2, 1 << 24, seed=24, offset=offset)


@pytest.mark.parametrize("dtype,N", [("bf16", 1), ("f32", 7), ("f16", 100), ("bf16", 1000), ("f32", 4096),
                                     ("bf16", 8192), ("f16", 20000)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_backward_forced_on_short_rows(monkeypatch, op, dtype, N):
    monkeypatch.setenv("MI355NORM_PATH", "split")
    go(op, dtype, 300, N, seed=N + 5)


@pytest.mark.parametrize("M,batch_rows", [(37, 5), (37, 1), (4500, 2000), (600, 600), (601, 600)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_backward_batches(monkeypatch, op, M, batch_rows):
    """Several batches: the first stores the partial rows, the later ones add
    to them; a last batch shorter than the row groups leaves the partial rows
    it does not reach as they were."""
    N = 2048
    monkeypatch.setenv("MI355NORM_PATH", "split")
    monkeypatch.setenv("MI355NORM_SPLIT_BATCH", str(batch_rows * 2 * N * 2))
    p = plan(op, M, N, "bf16")
    assert p["batch_rows"] == batch_rows
    go(op, "bf16", M, N, seed=M + batch_rows)


def test_split_backward_more_rows_than_the_row_sum_grid(monkeypatch):
    """More than 2^22 rows: the row-sum kernel's grid (2^20 workgroups of
    four wavefronts) walks the rows grid-strided."""
    monkeypatch.setenv("MI355NORM_PATH", "split")
    go("ln", "f32", (1 << 22) + 1000, 2, seed=99)


@pytest.mark.parametrize("grid", [1, 3, 1000])
def test_split_backward_forced_sums_grid(monkeypatch, grid):
    """The chunk-sum kernel's grid far below its work items (rows x chunks):
    the same bits as the full grid."""
    monkeypatch.setenv("MI355NORM_PATH", "split")
    for op in ("ln", "rms"):
        dy, x, g, mean, rstd = inputs(op, "bf16", 77, 40000, grid)
        ref = gpu_runner.run_bwd(op, "bf16", dy, x, g, mean, rstd)
        monkeypatch.setenv("MI355NORM_GRID", str(grid))
        _, got = go(op, "bf16", 77, 40000, seed=grid)
        monkeypatch.delenv("MI355NORM_GRID")
        for u, v in zip(ref, got):
            assert (u is None and v is None) or np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("dtype,N", [("bf16", 40000), ("f32", 20000), ("f16", 50001)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_backward_unaligned_pointers(op, dtype, N):
    go(op, dtype, 16, N, seed=N + 9, offset=1)


@pytest.mark.parametrize("which", ["dy", "x"])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_backward_in_place(op, which):
    _, (dx0, dg0, db0) = go(op, "bf16", 40, 40000, seed=3)
    _, (dx1, dg1, db1) = go(op, "bf16", 40, 40000, seed=3, inplace=which)
    assert np.array_equal(dx0, dx1) and np.array_equal(dg0, dg1)
    if op == "ln":
        assert np.array_equal(db0, db1)


@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_backward_optional_outputs_and_gamma(op):
    M, N = 20, 40000
    dy, x, g, mean, rstd = inputs(op, "f32", M, N, 11)
    for gamma, want_g, want_b in [(None, True, True), (g, False, True), (g, True, False), (g, False, False)]:
        print(f"[bwd split] optional gamma={gamma is not None} dg={want_g} db={want_b}", flush=True)
        dx, dg, db = gpu_runner.run_bwd(op, "f32", dy, x, gamma, mean, rstd, want_g=want_g, want_b=want_b)
        parity.check_bwd(op, "f32", dy, x, gamma, mean, rstd, dx, dg, db, plan(op, M, N, "f32"),
                         what=f"gamma={gamma is not None} dg={want_g} db={want_b}")
        assert (dg is None) == (not want_g)


def test_split_backward_no_rows_gives_zero_sums(monkeypatch):
    monkeypatch.setenv("MI355NORM_PATH", "split")
    for N in (1000, 40000):
        dg = torch.full((N,), float("nan"), device="cuda")
        db = torch.full((N,), float("nan"), device="cuda")
        st = rn.ln_bwd(None, None, None, None, None, None, dg.data_ptr(), db.data_ptr(), 0, N, rn.NORM_F32,
                       torch.cuda.current_stream().cuda_stream)
        assert st == rn.NORM_OK
        torch.cuda.synchronize()
        assert torch.all(dg == 0) and torch.all(db == 0)


@pytest.mark.parametrize("dtype,N,lddy,ldx,lddx,offset", [
    ("bf16", 40000, 40000 + 64, 40000 + 8, 40000 + 128, 0),     # 16-byte aligned rows
    ("bf16", 40000, 40000 + 3, 40000, 40000 + 5, 0),            # unaligned strides: element-wise
    ("f32", 33000, 33000 + 4, 33000 + 12, 33000 + 36, 1),
])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_split_backward_strided_rows(op, dtype, N, lddy, ldx, lddx, offset):
    M = 7
    dy, x, g, mean, rstd = inputs(op, dtype, M, N, N + 61)
    aligned = offset == 0 and all((v * E[dtype]) % 16 == 0 for v in (N, lddy, ldx, lddx))
    p = plan(op, M, N, dtype, aligned)
    assert p["path"] == "bwd_split"
    print(f"[bwd split] strided {op} {dtype} N={N} ld={lddy},{ldx},{lddx} offset={offset}", flush=True)
    dx, dg, db = gpu_runner.run_bwd_strided(op, dtype, dy, x, g, mean, rstd, lddy=lddy, ldx=ldx, lddx=lddx,
                                            offset=offset)
    parity.check_bwd(op, dtype, dy, x, g, mean, rstd, dx, dg, db, p, what=f"split strided {op}")


def test_split_backward_is_bitwise_deterministic():
    dy, x, g, mean, rstd = inputs("ln", "bf16", 300, 65536, 21)
    a = gpu_runner.run_bwd("ln", "bf16", dy, x, g, mean, rstd)
    b = gpu_runner.run_bwd("ln", "bf16", dy, x, g, mean, rstd)
    for u, v in zip(a, b):
        assert (u is None and v is None) or np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_split_agrees_with_row_kernel(monkeypatch):
    """The same rows through both paths: dx and the column sums within the
    oracle's bound of each other (their sums are taken in different orders)."""
    op, dtype, M, N = "ln", "bf16", 500, 8192
    dy, x, g, mean, rstd = inputs(op, dtype, M, N, 77)
    rows = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd)
    monkeypatch.setenv("MI355NORM_PATH", "split")
    p = plan(op, M, N, dtype)
    split = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd)
    parity.check_bwd(op, dtype, dy, x, g, mean, rstd, *split, p, what="split")
    assert not np.array_equal(rows[0], np.zeros_like(rows[0]))
    d = np.abs(oracle.widen(rows[0], dtype) - oracle.widen(split[0], dtype))
    assert d.max() <= 4 * parity.ulp_of(np.abs(oracle.widen(rows[0], dtype)).max(), dtype)


# ---------------------------------------------------------------------------
# the single pass (MI355NORM_PATH=splitpass)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,N,M", [("bf16", 40000, 24), ("f16", 65544, 9), ("bf16", 1 << 20, 6),
                                       ("f32", 1 << 20, 5), ("bf16", 30001, 17), ("f32", 1000, 300),
                                       ("bf16", 8192, 700), ("f16", 7, 50)])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_single_pass_split_backward(monkeypatch, op, dtype, N, M):
    """Every chunk of a row in its own workgroup, the chunk sums exchanged
    through the row's slots, dy and x read once; rows past the team count are
    walked by the teams."""
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    aligned = (N * E[dtype]) % 16 == 0
    p = plan(op, M, N, dtype, aligned)
    assert p["mode"] == "pass", p
    go(op, dtype, M, N, seed=N + M)


def test_single_pass_split_backward_chosen_automatically():
    """Without an override the backward takes the single pass for rows of
    16-byte vectors that leave the row kernel (and fp32 rows of 32 elements
    per lane) when a row's chunks fit at once and every team walks at least
    32 rows; fewer rows per team, or LayerNorm with fp16 I/O, keep the three
    kernels, and shorter rows the row kernel."""
    mode = lambda op, dtype, M, N: plan(op, M, N, dtype).get("mode", "rows")
    assert mode("ln", "bf16", 4096, 40000) == "pass"
    assert mode("rms", "f16", 2048, 65536) == "pass"
    assert mode("ln", "f32", 8192, 20000) == "pass"
    assert mode("rms", "f32", 2048, 32768) == "pass"
    assert mode("ln", "bf16", 64, 1 << 20) == "three"          # 16 rows per team
    assert mode("ln", "f16", 4096, 40000) == "three"
    assert mode("ln", "bf16", 4096, 40000 + 1) == "three"      # not 16-byte vectors
    assert mode("ln", "f32", 16384, 8192) == "rows"
    assert mode("ln", "bf16", 4096, 32768) == "rows"


@pytest.mark.parametrize("op", ["ln", "rms"])
def test_single_pass_split_backward_automatic_shape(op):
    """An fp32 shape the planner sends to the single pass by itself (64
    teams of 4 chunks over 2048 rows), every row and column against the
    oracle."""
    M, N = 2048, 32768
    p = plan(op, M, N, "f32")
    assert p["mode"] == "pass" and p["partial_rows"] * 32 <= M, p
    go(op, "f32", M, N, seed=77)


def test_single_pass_split_backward_in_place_and_deterministic(monkeypatch):
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    _, (dx0, dg0, db0) = go("ln", "bf16", 40, 70000, seed=5)
    _, (dx1, dg1, db1) = go("ln", "bf16", 40, 70000, seed=5)
    _, (dx2, dg2, db2) = go("ln", "bf16", 40, 70000, seed=5, inplace="dy")
    for a, b in ((dx0, dx1), (dg0, dg1), (db0, db1), (dx0, dx2), (dg0, dg2), (db0, db2)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("op,dtype,M,N", [("ln", "bf16", 6, 1 << 18), ("rms", "f32", 5, 70001), ("ln", "f16", 40, 40000),
                                         ("rms", "bf16", 6, 1 << 18)])
def test_single_pass_split_backward_recompute_gives_the_same_bits(monkeypatch, op, dtype, M, N):
    """The bounded wait, forced from the host to give up at once: every
    workgroup computes its rows' chunk sums from dy and x itself.  dx, dgamma
    and dbeta must be the normal single pass's bits, and the next normal call
    (slots and counters back at zero) must give them again."""
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    dy, x, g, mean, rstd = inputs(op, dtype, M, N, 62 + M)
    print(f"[bwd pass] {op} {dtype} M={M} N={N}: normal, recompute, normal", flush=True)
    a = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd)
    monkeypatch.setenv("MI355NORM_FORCE_TIMEOUT", "1")
    b = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd)
    monkeypatch.delenv("MI355NORM_FORCE_TIMEOUT")
    c = gpu_runner.run_bwd(op, dtype, dy, x, g, mean, rstd)
    for u, v, w in zip(a, b, c):
        if u is None:
            continue
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "recompute path differs"
        assert np.array_equal(u.view(np.uint8), w.view(np.uint8)), "call after the recompute differs"
    go(op, dtype, M, N, seed=62 + M)


@pytest.mark.parametrize("dtype,N,lddy,ldx,lddx,offset", [
    ("bf16", 40000, 40000 + 64, 40000 + 8, 40000 + 128, 0),
    ("bf16", 40000, 40000 + 3, 40000, 40000 + 5, 0),
    ("f32", 33000, 33000 + 4, 33000 + 12, 33000 + 36, 1),
])
@pytest.mark.parametrize("op", ["ln", "rms"])
def test_single_pass_split_backward_strided_rows(monkeypatch, op, dtype, N, lddy, ldx, lddx, offset):
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    M = 7
    dy, x, g, mean, rstd = inputs(op, dtype, M, N, N + 67)
    aligned = offset == 0 and all((v * E[dtype]) % 16 == 0 for v in (N, lddy, ldx, lddx))
    p = plan(op, M, N, dtype, aligned)
    assert p["mode"] == "pass"
    print(f"[bwd pass] strided {op} {dtype} N={N} ld={lddy},{ldx},{lddx} offset={offset}", flush=True)
    dx, dg, db = gpu_runner.run_bwd_strided(op, dtype, dy, x, g, mean, rstd, lddy=lddy, ldx=ldx, lddx=lddx,
                                            offset=offset)
    parity.check_bwd(op, dtype, dy, x, g, mean, rstd, dx, dg, db, p, what=f"pass strided {op}")


@pytest.mark.parametrize("op", ["ln", "rms"])
def test_single_pass_split_backward_optional_outputs_and_gamma(monkeypatch, op):
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    M, N = 20, 40000
    dy, x, g, mean, rstd = inputs(op, "f32", M, N, 13)
    for gamma, want_g, want_b in [(None, True, True), (g, False, True), (g, True, False), (g, False, False)]:
        print(f"[bwd pass] optional gamma={gamma is not None} dg={want_g} db={want_b}", flush=True)
        dx, dg, db = gpu_runner.run_bwd(op, "f32", dy, x, gamma, mean, rstd, want_g=want_g, want_b=want_b)
        parity.check_bwd(op, "f32", dy, x, gamma, mean, rstd, dx, dg, db, plan(op, M, N, "f32"),
                         what=f"pass gamma={gamma is not None} dg={want_g} db={want_b}")


@pytest.mark.parametrize("mode", ["split", "splitpass"])
def test_split_backward_unaligned_column_sums(monkeypatch, mode):
    """One row group writes dgamma / dbeta itself (batches of one row force
    it on the three-kernel form; one team on the single pass): with those
    outputs only 4-byte aligned the writes fall back from 16-byte vectors to
    single elements and still add up every batch."""
    monkeypatch.setenv("MI355NORM_PATH", mode)
    if mode == "split":
        M, N = 5, 2048
        monkeypatch.setenv("MI355NORM_SPLIT_BATCH", str(2 * N * 2))     # one row per batch
    else:
        M, N = 3, 3 << 20                                               # 192 chunks: one team
    dy, x, g, mean, rstd = inputs("ln", "bf16", M, N, 91)
    p = plan("ln", M, N, "bf16")
    if p["partial_rows"] != 1:
        pytest.skip(f"this device plans {p['partial_rows']} row groups here")
    dyt, xt, gt = (gpu_runner.to_device(a, "bf16") for a in (dy, x, g))
    mt, rt = torch.from_numpy(mean).cuda(), torch.from_numpy(rstd).cuda()
    dxt = torch.empty(M * N, dtype=torch.bfloat16, device="cuda")
    buf = torch.full((2 * N + 8,), float("nan"), device="cuda")
    dgt, dbt = buf[1:N + 1], buf[N + 5:2 * N + 5]          # 4-byte aligned, not 16
    assert dgt.data_ptr() % 16 and dbt.data_ptr() % 16
    print(f"[bwd {mode}] unaligned dgamma/dbeta {p}", flush=True)
    st = rn.ln_bwd(dyt.data_ptr(), xt.data_ptr(), gt.data_ptr(), mt.data_ptr(), rt.data_ptr(), dxt.data_ptr(),
                   dgt.data_ptr(), dbt.data_ptr(), M, N, rn.NORM_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_OK
    torch.cuda.synchronize()
    dx = gpu_runner.to_host(dxt, "bf16").reshape(M, N)
    parity.check_bwd("ln", "bf16", dy, x, g, mean, rstd, dx, dgt.cpu().numpy(), dbt.cpu().numpy(), p,
                     what=f"{mode} unaligned column sums")
