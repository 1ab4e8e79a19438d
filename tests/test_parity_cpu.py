"""The comparison rules of tests/parity.py, exercised on the CPU with
hand-made codes: exact agreement, tolerated near-tie neighbours, and the
differences that must fail."""
import numpy as np
import pytest

import oracle
import parity


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
