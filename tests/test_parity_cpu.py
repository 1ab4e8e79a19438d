"""The comparison rules of tests/parity.py, exercised on the CPU with
hand-made codes: exact agreement, tolerated near-tie neighbours, and the
differences that must fail."""
import numpy as np
import pytest

import oracle
import parity
import workloads


def codes(v, scale=1.0):
    return oracle.quant_e4m3(np.asarray(v, np.float64), scale)


def test_fp8_exact_agreement_and_zero_nan_signs():
    y = np.array([1.0, -3.25, 0.0, np.nan, 500.0])
    qr = codes(y)
    q = qr.copy()
    q[2] = 0x80                     # -0 for +0
    q[3] = 0xFF                     # NaN of the other sign
    assert parity.check_fp8(q, qr, y, 1.0)["fp8_near_ties"] == 0


def test_fp8_near_tie_neighbour_is_tolerated():
    # 1.0625 is the midpoint of 1.0 (0x38) and 1.125 (0x39): a value a few
    # fp32 ulps from it may round either way
    y = np.full(4000, 1.0)
    y[0] = 1.0625 * (1 + 1e-7)
    qr = codes(y)
    q = qr.copy()
    q[0] = 0x38
    assert qr[0] == 0x39
    assert parity.check_fp8(q, qr, y, 1.0)["fp8_near_ties"] == 1


def test_fp8_far_or_non_neighbour_differences_fail():
    y = np.full(4000, 1.0)
    y[0] = 1.07                      # well away from the midpoint
    qr = codes(y)
    q = qr.copy()
    q[0] = 0x38
    with pytest.raises(AssertionError):
        parity.check_fp8(q, qr, y, 1.0)
    y[0] = 1.0625 * (1 + 1e-7)
    qr = codes(y)
    q = qr.copy()
    q[0] = 0x37                      # two codes away
    with pytest.raises(AssertionError):
        parity.check_fp8(q, qr, y, 1.0)


def test_fp8_too_many_ties_fail():
    y = np.full(100, 1.0625 * (1 + 1e-7))
    qr = codes(y)
    q = np.full(100, 0x38, np.uint8)
    with pytest.raises(AssertionError):
        parity.check_fp8(q, qr, y, 1.0)


@pytest.mark.parametrize("op", ["ln", "rms"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_bound_accepts_the_rounded_oracle_and_rejects_a_dropped_term(op, dtype):
    M, N = 40, 96
    d = workloads.gen_bwd(3, M, N, dtype, op + "_bwd")
    if op == "ln":
        _, mean, rstd = oracle.ln_fwd(d["x"], d["gamma"], None, dtype, 1e-5)
        mean = mean.astype(np.float32)
        dx, dg, db = oracle.ln_bwd(d["dy"], d["x"], d["gamma"], dtype, mean, rstd.astype(np.float32))
    else:
        _, rstd = oracle.rms_fwd(d["x"], d["gamma"], dtype, 1e-6)
        mean, db = None, None
        dx, dg = oracle.rms_bwd(d["dy"], d["x"], d["gamma"], dtype, rstd.astype(np.float32))
    rstd = rstd.astype(np.float32)
    plan = {"work": M, "grid": 8, "rows_per_wg": 1}
    store = (lambda v: v.astype(np.float32)) if dtype == "f32" else (lambda v: oracle.round_to(v, dtype))
    parity.check_bwd(op, dtype, d["dy"], d["x"], d["gamma"], mean, rstd, store(dx), dg.astype(np.float32),
                     None if db is None else db.astype(np.float32), plan)
    # dx without its mean-of-g term (LayerNorm) or its rstd^3 term (RMSNorm) must fail
    g = oracle.widen(d["dy"], dtype) * oracle.widen(d["gamma"], dtype)
    if op == "ln":
        wrong = dx + rstd.astype(np.float64)[:, None] * g.mean(1, keepdims=True)
    else:
        xs = oracle.widen(d["x"], dtype)
        r = rstd.astype(np.float64)[:, None]
        wrong = dx + xs * r ** 3 * (g * xs).mean(1, keepdims=True)
    with pytest.raises(AssertionError, match="dx mismatch"):
        parity.check_bwd(op, dtype, d["dy"], d["x"], d["gamma"], mean, rstd, store(wrong), None, None, plan)
    # a column sum off by one row's term must fail
    bad = dg.astype(np.float32).copy()
    bad[5] += 1e-2
    with pytest.raises(AssertionError, match="dgamma"):
        parity.check_bwd(op, dtype, d["dy"], d["x"], d["gamma"], mean, rstd, store(dx), bad, None, plan)
