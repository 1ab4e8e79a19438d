"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Every check takes an `oracle.Oracle` instance and raises AssertionError when
the oracle disagrees.  `tests/test_oracle_pins.py` runs them on the real
oracle; `tests/test_oracle_mutants.py` runs them on deliberately broken builds
of oracle.c and requires each broken build to fail at least one of them.

Kinds of pins used:
  * printed values   -- the large-mean example row of "CUDA 算子工程" ch. 7,
                        section 7.3, and the N=5 padding example of
                        "T3 讲解" part ②  (tests/golden/*.txt);
  * exact brute force -- Fraction arithmetic for means and variances and a
                        50-digit Decimal square root, on tiny rows;
  * invariants       -- normalised rows have mean 0 and variance
                        var/(var+eps); RMS-normalised rows have mean square
                        ms/(ms+eps);
  * special cases    -- N=1, constant rows, eps=0; a zero residual makes
                        the residual-add step a plain RMSNorm;
  * library routines -- float64 torch layer_norm / rms_norm on the CPU,
                        numpy mean / var(ddof=0), numpy's double->half
                        conversion, torch's bfloat16 conversions.
"""
from __future__ import annotations

import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U64 = 2.0 ** -53


def read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals = [float(t) for t in v.split()]
            out[k] = vals[0] if len(vals) == 1 else vals
    return out


# --------------------------------------------------------------------------
# exact brute force (independent of the oracle's code)
# --------------------------------------------------------------------------

def exact_values(a: np.ndarray, dtype: str) -> list:
    """Exact rational value of each stored element, via library conversions."""
    if dtype in ("f32", "f64"):
        return [Fraction(float(v)) for v in a.ravel()]
    if dtype == "f16":
        return [Fraction(float(v)) for v in a.ravel().astype(np.float64)]
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(a.ravel().view(np.int16).copy()).view(torch.bfloat16)
        return [Fraction(float(v)) for v in t.to(torch.float64).numpy()]
    raise ValueError(dtype)


def _dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def brute_ln_row(x, g, b, eps):
    """Exact mean and variance (Fraction), rstd and y in 50-digit Decimal."""
    getcontext().prec = 50
    n = len(x)
    mu = sum(x, Fraction(0)) / n
    var = sum(((v - mu) ** 2 for v in x), Fraction(0)) / n
    if var + eps == 0:
        return mu, var, None, None       # rstd = inf, y = NaN (0 * inf)
    rs = Decimal(1) / _dec(var + Fraction(eps)).sqrt()
    y = [_dec(x[i] - mu) * rs * _dec(g[i]) + _dec(b[i]) for i in range(n)]
    return mu, var, rs, y


def brute_rms_row(x, g, eps):
    getcontext().prec = 50
    n = len(x)
    ms = sum((v * v for v in x), Fraction(0)) / n
    rs = Decimal(1) / _dec(ms + Fraction(eps)).sqrt()
    y = [_dec(x[i]) * rs * _dec(g[i]) for i in range(n)]
    return ms, rs, y


def _rel(a: float, b: float) -> float:
    return abs(a - b) / max(abs(b), 1e-300)


# --------------------------------------------------------------------------
# pins from the pages
# --------------------------------------------------------------------------

def pin_large_mean_row_decimal(orc):
    """Decimal example row of ch. 7 section 7.3: mean 1000.0055, var 8.25e-6."""
    g = read_golden("large_mean_row.txt")
    x = np.array(g["x"], np.float64).reshape(1, -1)
    xs = [Fraction(s) for s in ("1000.%03d" % k for k in range(1, 11))]
    # the fixture's closed forms, in exact decimal arithmetic
    assert sum(xs) == Fraction("10000.055")
    assert sum(v * v for v in xs) == Fraction("10000110.000385")
    assert sum(xs) / 10 == Fraction(str(g["mean"]))
    mu = sum(xs) / 10
    assert mu * mu == Fraction("1000011.00003025")
    assert sum((v - mu) ** 2 for v in xs) == Fraction(str(g["sum_dev_sq"]))
    # oracle on the row stored as doubles (eps = 0 so var = 1 / rstd^2)
    _, mean, rstd = orc.ln_fwd(x, None, None, "f64", 0.0, exact_eps=True)
    assert _rel(mean[0], g["mean"]) < 1e-14, mean[0]
    var = 1.0 / rstd[0] ** 2
    assert _rel(var, g["var"]) < 1e-9, var


def pin_large_mean_row_fp32(orc):
    """Same row stored in fp32: oracle equals the exact rational statistics."""
    from workloads import check_row_f32
    x = check_row_f32()
    xs = exact_values(x, "f32")
    mu, var, rs, y = brute_ln_row(xs, [Fraction(1)] * 10, [Fraction(0)] * 10,
                                  Fraction(float(np.float32(1e-5))))
    yo, mean, rstd = orc.ln_fwd(x, None, None, "f32", 1e-5)
    assert _rel(mean[0], float(mu)) < 1e-15
    assert _rel(rstd[0], float(rs)) < 1e-12
    # error of y in double is about u64 * |mu| * rstd (mu is not exact in double)
    tol = 64 * U64 * 2000.0 * float(rs)
    for i in range(10):
        assert abs(yo[0, i] - float(y[i])) <= tol, (i, yo[0, i], float(y[i]))
    # the spacing facts the fixture records
    g = read_golden("large_mean_row.txt")
    assert float(np.spacing(np.float32(1000.0))) == g["fp32_spacing_near_1000"]
    assert float(np.spacing(np.float32(1.0e6))) == g["fp32_spacing_near_1e6"]


def pin_naive_formula_fails(orc):
    """Negative control: E[x^2]-E[x]^2 in fp32 gives 0 or 0.25 on the row
    (ch. 7 section 7.3), far from the oracle's variance."""
    from workloads import check_row_f32
    g = read_golden("large_mean_row.txt")
    x = check_row_f32()[0]

    def naive(order):
        s = np.float32(0.0)
        q = np.float32(0.0)
        for v in order:
            s = np.float32(s + v)
            q = np.float32(q + np.float32(v * v))
        m = np.float32(s / np.float32(10.0))
        return float(np.float32(np.float32(q / np.float32(10.0)) - np.float32(m * m)))

    got = {naive(x), naive(x[::-1])}
    assert got <= set(g["naive_fp32_results"]), got
    _, _, rstd = orc.ln_fwd(x.reshape(1, -1), None, None, "f32", 0.0)
    var = 1.0 / rstd[0] ** 2
    for v in got:
        assert abs(v - var) >= 0.5 * var          # both results are useless
    # the page puts the 0.25 result at roughly thirty thousand times the truth
    assert 2.5e4 < 0.25 / var < 3.5e4


def pin_padding_n5(orc):
    """N=5 example of "T3 讲解" part ②: variance 1.2; unmasked padding 10.8."""
    g = read_golden("padding_n5.txt")
    x = np.array(g["x"], np.float64).reshape(1, -1)
    _, mean, rstd = orc.ln_fwd(x, None, None, "f64", 0.0, exact_eps=True)
    assert _rel(1.0 / rstd[0] ** 2, g["var"]) < 1e-14
    assert mean[0] == 4.0
    # negative control: pad to the block with zeros, centre without masking
    pad = np.zeros(int(g["block"]))
    pad[:5] = x[0]
    mu = pad.sum() / 5
    wrong = ((pad - mu) ** 2).sum() / 5
    assert abs(wrong - g["var_unmasked"]) < 1e-12
    assert abs(wrong - 1.0 / rstd[0] ** 2) > 1.0


# --------------------------------------------------------------------------
# exact brute force on tiny rows
# --------------------------------------------------------------------------

def _tiny_cases(seed=7):
    rng = np.random.default_rng(seed)
    cases = []
    for dtype in ("f32", "bf16", "f16"):
        for n in (1, 2, 3, 5, 8, 13, 16):
            loc = float(rng.choice([0.0, 3.0, -50.0, 1000.0]))
            scale = float(rng.choice([1.0, 0.01, 7.0]))
            x = (loc + scale * rng.standard_normal((2, n))).astype(np.float32)
            gm = rng.uniform(-1.5, 1.5, n).astype(np.float32)
            bt = rng.normal(0, 0.5, n).astype(np.float32)
            eps = float(rng.choice([1e-5, 1e-6, 0.25, 0.0]))
            from workloads import to_storage
            cases.append((dtype, to_storage(x, dtype), to_storage(gm, dtype),
                          to_storage(bt, dtype), eps))
    return cases


def pin_brute_force_ln(orc):
    for dtype, x, gm, bt, eps in _tiny_cases():
        xs_all = exact_values(x, dtype)
        gs = exact_values(gm, dtype)
        bs = exact_values(bt, dtype)
        n = x.shape[1]
        e = Fraction(float(np.float32(eps)))
        y, mean, rstd = orc.ln_fwd(x, gm, bt, dtype, eps)
        for r in range(x.shape[0]):
            xs = xs_all[r * n:(r + 1) * n]
            mu, var, rs, yb = brute_ln_row(xs, gs, bs, e)
            if rs is None:
                assert np.isinf(rstd[r]) and np.all(np.isnan(y[r])), (dtype, n, r)
                continue
            amax = max(abs(float(v)) for v in xs)
            assert abs(mean[r] - float(mu)) <= 4 * n * U64 * amax + 1e-300, (dtype, n, r)
            kappa = amax / max(float(var) ** 0.5, 1e-300)
            assert _rel(rstd[r], float(rs)) <= 32 * n * U64 * (1 + kappa * kappa * n * U64) + 1e-15, \
                (dtype, n, r, rstd[r], float(rs))
            for i in range(n):
                tol = 64 * U64 * ((abs(float(xs[i])) + abs(float(mu))) * float(rs) * abs(float(gs[i]))
                                  + abs(float(bs[i])) + abs(float(yb[i])))
                assert abs(y[r, i] - float(yb[i])) <= tol + 1e-300, (dtype, n, r, i)


def pin_brute_force_rms(orc):
    for dtype, x, gm, _, eps in _tiny_cases(seed=11):
        xs_all = exact_values(x, dtype)
        gs = exact_values(gm, dtype)
        n = x.shape[1]
        e = Fraction(float(np.float32(eps)))
        y, rstd = orc.rms_fwd(x, gm, dtype, eps)
        for r in range(x.shape[0]):
            xs = xs_all[r * n:(r + 1) * n]
            ms, rs, yb = brute_rms_row(xs, gs, e)
            assert _rel(rstd[r], float(rs)) <= 16 * n * U64, (dtype, n, r)
            for i in range(n):
                assert abs(y[r, i] - float(yb[i])) <= 16 * n * U64 * abs(float(yb[i])) + 1e-300


# --------------------------------------------------------------------------
# invariants and special cases
# --------------------------------------------------------------------------

def pin_invariants(orc):
    rng = np.random.default_rng(3)
    for n in (7, 64, 1000, 4096):
        x = (5.0 + 3.0 * rng.standard_normal((4, n))).astype(np.float32)
        y, mean, rstd = orc.ln_fwd(x, None, None, "f32", 0.0)
        for r in range(4):
            assert abs(y[r].mean()) <= 1e-12 * np.abs(y[r]).max()
            assert abs(y[r].var() - 1.0) <= 1e-12
        eps = 0.5
        y, mean, rstd = orc.ln_fwd(x, None, None, "f32", eps)
        v = x.astype(np.float64).var(axis=1)
        for r in range(4):
            assert _rel(y[r].var(), v[r] / (v[r] + eps)) <= 1e-12
        y, rstd = orc.rms_fwd(x, None, "f32", 0.0)
        for r in range(4):
            assert abs((y[r] ** 2).mean() - 1.0) <= 1e-12
        y, rstd = orc.rms_fwd(x, None, "f32", eps)
        ms = (x.astype(np.float64) ** 2).mean(axis=1)
        for r in range(4):
            assert _rel((y[r] ** 2).mean(), ms[r] / (ms[r] + eps)) <= 1e-12


def pin_special_cases(orc):
    gm = np.array([1.5], np.float32)
    bt = np.array([-0.25], np.float32)
    x = np.array([[3.0], [-7.5]], np.float32)
    eps = 1e-5
    e = float(np.float32(eps))
    y, mean, rstd = orc.ln_fwd(x, gm, bt, "f32", eps)
    assert np.all(y == -0.25)                          # N = 1: y = beta
    assert np.all(mean == x[:, 0])
    assert np.all(np.abs(rstd - 1.0 / np.sqrt(e)) <= 1e-15 * rstd)
    # constant row: y = beta, rstd = 1/sqrt(eps)
    xc = np.full((1, 9), 42.0, np.float32)
    gc = np.linspace(0.5, 1.5, 9).astype(np.float32)
    bc = np.linspace(-1, 1, 9).astype(np.float32)
    y, mean, rstd = orc.ln_fwd(xc, gc, bc, "f32", eps)
    assert np.array_equal(y[0], bc.astype(np.float64))
    assert mean[0] == 42.0
    # eps = 0 on a constant row: rstd = inf, y = NaN (IEEE 0 * inf)
    y, mean, rstd = orc.ln_fwd(xc, None, None, "f32", 0.0)
    assert np.isinf(rstd[0]) and np.all(np.isnan(y))
    # RMS with N = 1: y = x / sqrt(x^2 + eps) * gamma
    y, rstd = orc.rms_fwd(x, gm, "f32", eps)
    for r in range(2):
        xv = float(x[r, 0])
        want = xv / np.sqrt(xv * xv + e) * 1.5
        assert _rel(y[r, 0], want) <= 1e-15
    # RMS of a zero row with eps = 0: NaN
    y, rstd = orc.rms_fwd(np.zeros((1, 4), np.float32), None, "f32", 0.0)
    assert np.isinf(rstd[0]) and np.all(np.isnan(y))


def pin_library_crosscheck(orc):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    for n in (1, 10, 257, 2048):
        x = (2.0 + rng.standard_normal((6, n))).astype(np.float32)
        gm = rng.uniform(0.5, 1.5, n).astype(np.float32)
        bt = rng.normal(0, 0.1, n).astype(np.float32)
        eps = 1e-5
        e = float(np.float32(eps))
        y, mean, rstd = orc.ln_fwd(x, gm, bt, "f32", eps)
        xt = torch.from_numpy(x).double()
        yt = F.layer_norm(xt, (n,), torch.from_numpy(gm).double(),
                          torch.from_numpy(bt).double(), e).numpy()
        assert np.max(np.abs(y - yt)) <= 1e-12
        x64 = x.astype(np.float64)
        assert np.max(np.abs(mean - x64.mean(axis=1))) <= 1e-12 * np.abs(x64).max()
        assert np.max(np.abs((1.0 / rstd ** 2 - e) - x64.var(axis=1))) <= 1e-12
        y, rstd = orc.rms_fwd(x, gm, "f32", 1e-6)
        yt = F.rms_norm(xt, (n,), torch.from_numpy(gm).double(), float(np.float32(1e-6))).numpy()
        assert np.max(np.abs(y - yt)) <= 1e-12


# --------------------------------------------------------------------------
# storage conversions
# --------------------------------------------------------------------------

def pin_widen_exhaustive(orc):
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = orc.widen(bits.view(np.float16), "f16")
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(h), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(h[m], ref[m])
    b = orc.widen(bits, "bf16")
    refb = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(b), np.isnan(refb))
    m = ~np.isnan(refb)
    assert np.array_equal(b[m], refb[m])


def _bf16_val(bits):
    w = np.array([int(bits) << 16], np.uint32)
    return float(w.view(np.float32)[0])


def pin_round_bf16(orc):
    import torch
    one = 1.0
    cases = [
        (one + 2.0 ** -8, 1.0),                               # tie -> even
        (one + 3 * 2.0 ** -8, one + 2.0 ** -6),               # tie -> even (up)
        (one + 2.0 ** -8 + 2.0 ** -40, one + 2.0 ** -7),      # no double rounding
        (-(one + 2.0 ** -8 + 2.0 ** -40), -(one + 2.0 ** -7)),
        (one + 2.0 ** -8 - 2.0 ** -40, 1.0),
        (2.0 ** -133, 2.0 ** -133),                           # smallest subnormal
        (2.0 ** -134, 0.0),                                   # tie -> even (zero)
        (1.5 * 2.0 ** -133, 2.0 ** -132),
        (255.0 * 2.0 ** 120, 255.0 * 2.0 ** 120),             # largest finite
        ((256.0 - 0.5) * 2.0 ** 120, float("inf")),           # tie at the top -> inf
        (1e300, float("inf")),
        (-1e300, float("-inf")),
        (99999.99, 99840.0),
        (1000.0 + 1.9, 1000.0),
        (1000.0 + 2.0, 1000.0),                               # tie -> even (1000 = 125*8)
        (1000.0 + 2.0 + 1e-9, 1004.0),
    ]
    v = np.array([c[0] for c in cases])
    out = orc.round_to(v, "bf16")
    for (inp, want), b in zip(cases, out):
        assert _bf16_val(b) == want, (inp, want, _bf16_val(b))
    # float32 inputs have no double-rounding issue: must agree with torch's RNE
    rng = np.random.default_rng(9)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.round_to(f.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def pin_round_f16_f32(orc):
    rng = np.random.default_rng(13)
    v = rng.standard_normal(50000) * np.exp2(rng.integers(-30, 18, 50000))
    # add exact ties and near-ties between binary16 neighbours
    base = np.arange(1, 2049, dtype=np.float64)
    ties = np.concatenate([(base + 0.5) * 2.0 ** -10, (base + 0.5) * 2.0 ** -24,
                           (base + 0.5) * 2.0 ** 5, -(base + 0.5) * 2.0 ** -3])
    v = np.concatenate([v, ties, np.nextafter(ties, 0), np.nextafter(ties, np.inf),
                        [65504.0, 65519.99, 65520.0, -65520.0, 0.0, -0.0, 2.0 ** -25,
                         3 * 2.0 ** -26]])
    got = orc.round_to(v, "f16")
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    got32 = orc.round_to(v, "f32")
    assert np.array_equal(got32, v.astype(np.float32))


# --------------------------------------------------------------------------
# residual add + RMSNorm
# --------------------------------------------------------------------------

FORMATS = {"f32": (24, -126), "bf16": (8, -126), "f16": (11, -14), "e4m3": (4, -6)}


def round_fraction(v: Fraction, dtype: str) -> Fraction:
    """Exact round-to-nearest-even of a rational to a binary format (finite
    results only), written from the definition: the quantum of v's binade
    (or of the smallest normal binade for subnormals), then the nearest
    multiple of it, ties to the even multiple."""
    prec, emin = FORMATS[dtype]
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - prec + 1)
    k = a / q
    f = k.numerator // k.denominator
    rem = k - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    r = f * q
    return r if v > 0 else -r


def _add_cases(seed=17):
    """Tiny rows whose sums mostly do not fit the storage type: x large,
    the residual small and not aligned to x's quantum."""
    from workloads import to_storage
    rng = np.random.default_rng(seed)
    cases = []
    for dtype in ("f32", "bf16", "f16"):
        for n in (1, 3, 8, 13):
            x = (rng.choice([1.0, 37.0, -300.0]) * (1 + rng.random((2, n)))).astype(np.float32)
            r = (rng.standard_normal((2, n)) * rng.choice([1e-3, 0.3, 3.0])).astype(np.float32)
            gm = rng.uniform(-1.5, 1.5, n).astype(np.float32)
            eps = float(rng.choice([1e-6, 0.5]))
            cases.append((dtype, to_storage(x, dtype), to_storage(r, dtype), to_storage(gm, dtype), eps))
    return cases


def pin_add_rms_brute_force(orc):
    """h = RNE(x + res) exactly (rational arithmetic), then the exact RMSNorm
    of h; at least some sums must need rounding, or the pin would not see a
    norm taken of the unrounded sum."""
    rounded = 0
    for dtype, x, r, gm, eps in _add_cases():
        xs = exact_values(x, dtype)
        rs_ = exact_values(r, dtype)
        gs = exact_values(gm, dtype)
        n = x.shape[1]
        h, y, rstd = orc.add_rms_fwd(x, r, gm, dtype, eps)
        hs = exact_values(h, dtype)
        e = Fraction(float(np.float32(eps)))
        for row in range(x.shape[0]):
            hb = []
            for i in range(n):
                k = row * n + i
                want = round_fraction(xs[k] + rs_[k], dtype)
                rounded += want != xs[k] + rs_[k]
                assert hs[k] == want, (dtype, n, row, i, hs[k], want)
                hb.append(want)
            ms, rsb, yb = brute_rms_row(hb, gs, e)
            assert _rel(rstd[row], float(rsb)) <= 16 * n * U64, (dtype, n, row)
            for i in range(n):
                assert abs(y[row, i] - float(yb[i])) <= 16 * n * U64 * abs(float(yb[i])) + 1e-300
    assert rounded > 20, rounded


def pin_add_rms_reduces_to_rms(orc):
    """A zero residual (or a zero x) makes the step a plain RMSNorm: h is the
    other operand bit for bit, and y, rstd equal rms_fwd's exactly; the add is
    commutative."""
    from workloads import to_storage
    rng = np.random.default_rng(19)
    for dtype in ("f32", "bf16", "f16"):
        x = to_storage((2.0 * rng.standard_normal((3, 40))).astype(np.float32), dtype)
        r = to_storage((0.7 * rng.standard_normal((3, 40))).astype(np.float32), dtype)
        gm = to_storage(rng.uniform(0.5, 1.5, 40).astype(np.float32), dtype)
        z = np.zeros_like(x)
        y0, rs0 = orc.rms_fwd(x, gm, dtype, 1e-6)
        for a, b in ((x, z), (z, x)):
            h, y, rstd = orc.add_rms_fwd(a, b, gm, dtype, 1e-6)
            assert np.array_equal(h.view(np.uint8), x.view(np.uint8)), dtype
            assert np.array_equal(y, y0) and np.array_equal(rstd, rs0), dtype
        h1, y1, r1 = orc.add_rms_fwd(x, r, gm, dtype, 1e-6)
        h2, y2, r2 = orc.add_rms_fwd(r, x, gm, dtype, 1e-6)
        assert np.array_equal(h1.view(np.uint8), h2.view(np.uint8))
        assert np.array_equal(y1, y2) and np.array_equal(r1, r2)


def pin_add_rms_library(orc):
    """h against the libraries' own storage-type addition (numpy float32 and
    float16, torch bfloat16), y against float64 torch rms_norm of h, on
    rows of realistic width."""
    import torch
    import torch.nn.functional as F
    from workloads import to_storage
    rng = np.random.default_rng(23)
    n = 1536
    xf = (rng.standard_normal((4, n)) * 3).astype(np.float32)
    rf = (rng.standard_normal((4, n)) * 0.05).astype(np.float32)
    gf = rng.uniform(0, 1, n).astype(np.float32)
    for dtype in ("f32", "f16", "bf16"):
        x, r, gm = to_storage(xf, dtype), to_storage(rf, dtype), to_storage(gf, dtype)
        h, y, rstd = orc.add_rms_fwd(x, r, gm, dtype, 1e-6)
        if dtype == "bf16":
            tb = lambda a: torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
            ref = (tb(x) + tb(r)).view(torch.int16).numpy().view(np.uint16)
            hd = tb(h).double()
            gd = tb(gm).double()
        else:
            ref = x + r                       # numpy adds in the storage type, RNE
            hd = torch.from_numpy(h.astype(np.float64))
            gd = torch.from_numpy(gm.astype(np.float64))
        assert np.array_equal(h.view(np.uint8), ref.view(np.uint8)), dtype
        yt = F.rms_norm(hd, (n,), gd, float(np.float32(1e-6))).numpy()
        assert np.max(np.abs(y - yt)) <= 1e-12, dtype


# --------------------------------------------------------------------------
# FP8 (OCP E4M3) output
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of an E4M3 code from the format's definition (NaN for
    S.1111.111): sign, 4-bit exponent with bias 7, 3-bit fraction."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    f = code & 7
    if e == 0xF and f == 7:
        return float("nan")
    if e == 0:
        return s * f / 8.0 * 2.0 ** -6
    return s * (1.0 + f / 8.0) * 2.0 ** (e - 7)


def e4m3_exact_code(v: Fraction) -> int:
    """Code of the saturated, round-to-nearest-even E4M3 value of a rational."""
    a = min(abs(v), Fraction(448))
    r = round_fraction(a, "e4m3")
    sign = 0x80 if v < 0 else 0
    for c in range(0x7F):                  # the 127 non-negative finite codes
        if Fraction(e4m3_value(c)) == r:
            return sign | c
    raise AssertionError(v)


def pin_e4m3_quantisation(orc):
    """Every code maps back to itself; midpoints between neighbours go to the
    even code; values past 448 saturate; the scale divides; NaN stays NaN;
    in-range values agree with torch's float8_e4m3fn conversion."""
    import torch
    vals = np.array([e4m3_value(c) for c in range(256)])
    codes = orc.quant_e4m3(vals, 1.0)
    for c in range(256):
        if np.isnan(vals[c]):
            assert codes[c] in (0x7F, 0xFF)
        else:
            assert codes[c] == c, (hex(c), hex(codes[c]))
    pos = [e4m3_value(c) for c in range(0x7F)]
    mids = np.array([(pos[i] + pos[i + 1]) / 2 for i in range(len(pos) - 1)])
    got = orc.quant_e4m3(mids, 1.0)
    for i, g in enumerate(got):
        assert g == (i if i % 2 == 0 else i + 1), (i, mids[i], hex(g))
    got = orc.quant_e4m3(np.nextafter(mids, np.inf), 1.0)
    assert np.array_equal(got, np.arange(1, 0x7F))
    got = orc.quant_e4m3(-np.nextafter(mids, 0), 1.0)
    assert np.array_equal(got, 0x80 | np.arange(0, 0x7E))
    big = orc.quant_e4m3(np.array([448.0, 463.9, 464.0, 1e6, np.inf, -500.0, -np.inf]), 1.0)
    assert list(big) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert orc.quant_e4m3(np.array([np.nan]), 1.0)[0] == 0x7F
    rng = np.random.default_rng(41)
    v = rng.standard_normal(5000) * np.exp2(rng.integers(-12, 8, 5000))
    for scale in (1.0, 0.0625, 3.0):
        got = orc.quant_e4m3(v, scale)
        w = torch.from_numpy(v / float(np.float32(scale)))
        ok = w.abs() <= 448
        ref = w[ok].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got[ok.numpy()], ref), scale
    two = orc.quant_e4m3(v, 2.0)
    assert np.array_equal(two, orc.quant_e4m3(v / 2.0, 1.0))


def pin_rms_fp8_brute_force(orc):
    """Codes of the exact RMSNorm output divided by the scale, saturated and
    rounded exactly, on tiny rows (both with and without the residual add)."""
    for dtype, x, gm, _, eps in _tiny_cases(seed=43):
        xs_all = exact_values(x, dtype)
        gs = exact_values(gm, dtype)
        n = x.shape[1]
        e = Fraction(float(np.float32(eps)))
        for scale in (0.01, 1.0, 0.3):
            sc = Fraction(float(np.float32(scale)))
            q, y, rstd = orc.rms_fp8_fwd(x, gm, dtype, eps, scale)
            for r in range(x.shape[0]):
                xs = xs_all[r * n:(r + 1) * n]
                _, rs, yb = brute_rms_row(xs, gs, e)
                for i in range(n):
                    want = e4m3_exact_code(Fraction(yb[i]) / sc)
                    assert q[r, i] == want or (want & 0x7F) == 0 and (q[r, i] & 0x7F) == 0, \
                        (dtype, n, r, i, hex(q[r, i]), hex(want))
    for dtype, x, res, gm, eps in _add_cases(seed=45):
        h, q, y, rstd = orc.add_rms_fp8_fwd(x, res, gm, dtype, eps, 0.05)
        hs = exact_values(h, dtype)
        gs = exact_values(gm, dtype)
        n = x.shape[1]
        for r in range(x.shape[0]):
            _, rs, yb = brute_rms_row(hs[r * n:(r + 1) * n], gs, Fraction(float(np.float32(eps))))
            for i in range(n):
                want = e4m3_exact_code(Fraction(yb[i]) / Fraction(float(np.float32(0.05))))
                assert q[r, i] == want, (dtype, n, r, i)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def _bwd_cases(seed=51):
    rng = np.random.default_rng(seed)
    out = []
    for n in (1, 2, 5, 16, 33):
        x = (rng.choice([0.0, 4.0, -30.0]) + rng.choice([1.0, 0.2]) * rng.standard_normal((3, n)))
        dy = rng.standard_normal((3, n))
        gm = rng.uniform(-1.5, 1.5, n)
        bt = rng.normal(0, 0.3, n)
        out.append((x, dy, gm, bt, float(rng.choice([1e-5, 0.1]))))
    return out


def pin_backward_finite_differences(orc):
    """Central differences of the (pinned) forward oracle: L = sum(dy * y),
    dL/dx, dL/dgamma, dL/dbeta against the backward oracle."""
    for x, dy, gm, bt, eps in _bwd_cases():
        M, n = x.shape
        _, mean, rstd = orc.ln_fwd(x, gm, bt, "f64", eps, exact_eps=True)
        dx, dg, db = orc.ln_bwd(dy, x, gm, "f64", mean, rstd)
        _, rr = orc.rms_fwd(x, gm, "f64", eps, exact_eps=True)
        rdx, rdg = orc.rms_bwd(dy, x, gm, "f64", rr)

        def L(xx, gg, bb, rms=False):
            if rms:
                return float((dy * orc.rms_fwd(xx, gg, "f64", eps, exact_eps=True)[0]).sum())
            return float((dy * orc.ln_fwd(xx, gg, bb, "f64", eps, exact_eps=True)[0]).sum())

        for rms, gx, gg, gb in ((False, dx, dg, db), (True, rdx, rdg, None)):
            scale = max(1.0, float(np.abs(gx).max()), float(np.abs(gg).max()))
            for r in range(M):
                for i in range(n):
                    h = 1e-6 * max(1.0, abs(x[r, i]))
                    xp, xm = x.copy(), x.copy()
                    xp[r, i] += h
                    xm[r, i] -= h
                    num = (L(xp, gm, bt, rms) - L(xm, gm, bt, rms)) / (2 * h)
                    assert abs(num - gx[r, i]) <= 1e-6 * scale, (rms, n, r, i, num, gx[r, i])
            for i in range(n):
                gp, gmn = gm.copy(), gm.copy()
                gp[i] += 1e-6
                gmn[i] -= 1e-6
                num = (L(x, gp, bt, rms) - L(x, gmn, bt, rms)) / 2e-6
                assert abs(num - gg[i]) <= 1e-6 * scale, (rms, n, i, num, gg[i])
                if gb is not None:
                    bp, bm = bt.copy(), bt.copy()
                    bp[i] += 1e-6
                    bm[i] -= 1e-6
                    num = (L(x, gm, bp) - L(x, gm, bm)) / 2e-6
                    assert abs(num - gb[i]) <= 1e-6 * scale, (n, i, num, gb[i])


def pin_backward_library_and_invariants(orc):
    """float64 torch autograd of layer_norm / rms_norm, and the invariants:
    LayerNorm dx sums to 0 over a row, and (eps = 0) dx is orthogonal to
    xhat; RMSNorm (eps = 0) dx is orthogonal to x."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(53)
    for n in (7, 256, 1000):
        x = (2.0 + rng.standard_normal((4, n))).astype(np.float32)
        dy = rng.standard_normal((4, n)).astype(np.float32)
        gm = rng.uniform(0.5, 1.5, n).astype(np.float32)
        bt = rng.normal(0, 0.1, n).astype(np.float32)
        e = float(np.float32(1e-5))
        _, mean, rstd = orc.ln_fwd(x, gm, bt, "f32", 1e-5)
        dx, dg, db = orc.ln_bwd(dy, x, gm, "f32", mean, rstd)
        xt = torch.from_numpy(x).double().requires_grad_()
        gt = torch.from_numpy(gm).double().requires_grad_()
        bt_ = torch.from_numpy(bt).double().requires_grad_()
        F.layer_norm(xt, (n,), gt, bt_, e).backward(torch.from_numpy(dy).double())
        assert np.max(np.abs(dx - xt.grad.numpy())) <= 1e-10
        assert np.max(np.abs(dg - gt.grad.numpy())) <= 1e-9 and np.max(np.abs(db - bt_.grad.numpy())) <= 1e-9
        assert np.max(np.abs(dx.sum(axis=1))) <= 1e-10 * np.abs(dx).max()
        _, r = orc.rms_fwd(x, gm, "f32", 1e-6)
        rdx, rdg = orc.rms_bwd(dy, x, gm, "f32", r)
        xt = torch.from_numpy(x).double().requires_grad_()
        gt = torch.from_numpy(gm).double().requires_grad_()
        F.rms_norm(xt, (n,), gt, float(np.float32(1e-6))).backward(torch.from_numpy(dy).double())
        assert np.max(np.abs(rdx - xt.grad.numpy())) <= 1e-10
        assert np.max(np.abs(rdg - gt.grad.numpy())) <= 1e-9
        # eps = 0 orthogonality
        _, mean0, rstd0 = orc.ln_fwd(x, gm, bt, "f32", 0.0)
        dx0, _, _ = orc.ln_bwd(dy, x, gm, "f32", mean0, rstd0)
        xhat = (x.astype(np.float64) - mean0[:, None]) * rstd0[:, None]
        assert np.max(np.abs((dx0 * xhat).sum(axis=1))) <= 1e-9 * np.abs(dx0).max() * n
        _, r0 = orc.rms_fwd(x, gm, "f32", 0.0)
        rdx0, _ = orc.rms_bwd(dy, x, gm, "f32", r0)
        assert np.max(np.abs((rdx0 * x).sum(axis=1))) <= 1e-9 * np.abs(rdx0 * x).max() * n


ALL_PINS = [
    pin_large_mean_row_decimal,
    pin_large_mean_row_fp32,
    pin_naive_formula_fails,
    pin_padding_n5,
    pin_brute_force_ln,
    pin_brute_force_rms,
    pin_invariants,
    pin_special_cases,
    pin_library_crosscheck,
    pin_widen_exhaustive,
    pin_round_bf16,
    pin_round_f16_f32,
    pin_add_rms_brute_force,
    pin_add_rms_reduces_to_rms,
    pin_add_rms_library,
    pin_e4m3_quantisation,
    pin_rms_fp8_brute_force,
    pin_backward_finite_differences,
    pin_backward_library_and_invariants,
]
