"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, rejects every bad argument with its status before any HIP call,
and plans the row-to-workgroup mapping as documented.  No kernel runs here."""
import ctypes
import os
import re

import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import rmsnorm_forward_amd as rn  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355norm.h")

OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_EPS, BAD_ARG, ALIAS, HIP = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["add_rms_fp8_fwd", "add_rms_fwd", "ln_bwd", "ln_fwd", "norm_bwd",
                                    "norm_bwd_describe", "norm_describe", "norm_fwd", "norm_fwd_noalloc", "norm_last_error",
                                    "norm_status_str", "rms_bwd", "rms_fp8_fwd", "rms_fwd"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(rn.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {rn.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_one_hip_runtime_in_the_process():
    # the library must bind to the HIP runtime torch loaded, not map a second
    import subprocess
    import sys
    code = ("import rmsnorm_forward_amd\n"
            "m = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         cwd=os.path.dirname(os.path.dirname(rn.LIB_PATH)))
    assert out.stdout.strip() == "1"


def test_status_strings():
    for code in range(9):
        s = rn.norm_status_str(code)
        assert s and s != "unknown status"
    assert rn.norm_status_str(99) == "unknown status"


def test_last_error_starts_empty():
    # the record is per thread: a new thread has seen no failure
    import threading
    seen = []
    t = threading.Thread(target=lambda: seen.append(rn.norm_last_error()))
    t.start()
    t.join()
    assert seen == [""]


# fake, never dereferenced device addresses: validation only does arithmetic
def _device_present() -> bool:
    """Whether a GPU is visible (device_count does not initialise HIP)."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


X, G, B, Y, MEAN, RSTD = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000

# calls that pass validation with the made-up addresses above go on to a
# launch: without a device it fails at once, with one it would read them
no_device_only = pytest.mark.skipif(_device_present(), reason="calls pass validation with made-up addresses; "
                                                             "they may only run where no device is present")


def call(op="ln", x=X, g=G, b=B, y=Y, mean=MEAN, rstd=RSTD, M=4, N=64, eps=1e-5, dtype=0):
    fn = rn.ln_fwd if op == "ln" else rn.rms_fwd
    if op == "rms" and b == B:
        b = None
    if op == "rms" and mean == MEAN:
        mean = None
    return fn(x, g, b, y, mean, rstd, M, N, eps, dtype, None)


@pytest.mark.parametrize("op", ["ln", "rms"])
def test_validation_paths(op):
    assert call(op, dtype=3) == BAD_DTYPE
    assert call(op, dtype=-1) == BAD_DTYPE
    assert call(op, M=-1) == BAD_SHAPE
    assert call(op, N=0) == BAD_SHAPE
    assert call(op, N=-5) == BAD_SHAPE
    assert call(op, N=(1 << 24) + 1) == BAD_SHAPE
    assert call(op, M=(1 << 62), N=1 << 20) == BAD_SHAPE
    assert call(op, eps=-1e-5) == BAD_EPS
    assert call(op, eps=float("nan")) == BAD_EPS
    assert call(op, eps=float("inf")) == BAD_EPS
    assert call(op, M=0, x=None, y=None) == OK          # nothing to do, nothing launched
    assert call(op, x=None) == NULL_ARG
    assert call(op, y=None) == NULL_ARG
    assert call(op, x=X + 2) == BAD_ARG                 # f32 element misaligned
    assert call(op, y=Y + 1, dtype=2) == BAD_ARG        # bf16 element misaligned
    assert call(op, rstd=RSTD + 2) == BAD_ARG
    assert call(op, y=X + 64) == ALIAS                  # y inside x
    assert call(op, y=X) == ALIAS                       # in place
    assert call(op, rstd=Y + 16) == ALIAS               # stats inside y
    assert call(op, g=Y + 4) == ALIAS                   # gamma inside y


R, H = 0x700000, 0x800000


def call_add(x=X, r=R, g=G, y=Y, h=H, rstd=RSTD, M=4, N=64, eps=1e-6, dtype=0):
    return rn.add_rms_fwd(x, r, g, y, h, rstd, M, N, eps, dtype, None)


def test_add_rms_validation():
    assert call_add(dtype=5) == BAD_DTYPE
    assert call_add(N=0) == BAD_SHAPE
    assert call_add(eps=-1.0) == BAD_EPS
    assert call_add(M=0, x=None, r=None, y=None, h=None) == OK
    assert call_add(r=None) == NULL_ARG
    assert call_add(h=None) == NULL_ARG
    assert call_add(x=None) == NULL_ARG
    assert call_add(r=R + 2) == BAD_ARG                 # misaligned residual
    assert call_add(h=H + 2) == BAD_ARG
    assert call_add(y=X + 64) == ALIAS                  # partial overlap is never allowed
    assert call_add(h=R + 16) == ALIAS
    assert call_add(h=Y) == ALIAS                       # the two outputs
    assert call_add(y=R + 4) == ALIAS
    assert call_add(g=H + 8) == ALIAS
    assert call_add(rstd=H) == ALIAS


@no_device_only
def test_add_rms_exact_in_place_passes_validation():
    # y over x and the sum over the residual (exactly the same pointers) are
    # allowed; without a GPU the call then fails at the first HIP call
    for kw in (dict(y=X), dict(h=R), dict(y=X, h=R), dict(y=R, h=X)):
        st = call_add(**kw)
        assert st not in (ALIAS, BAD_ARG, NULL_ARG), (kw, st)


def test_add_rms_plans_like_rms():
    # the same tiles up to 512 vectors a row and on split rows; past that
    # plain RMSNorm with 16-bit I/O takes two vectors per lane, the residual
    # add four
    for N in (1024, 2048, 4096, 1 << 20):
        a = parse(rn.norm_describe("add_rms", 64, N, "bf16"))
        b = parse(rn.norm_describe("rms", 64, N, "bf16"))
        assert a == b, (N, a, b)
    for N in (8192, 16384):
        a = parse(rn.norm_describe("add_rms", 64, N, "bf16"))
        b = parse(rn.norm_describe("rms", 64, N, "bf16"))
        assert (a["vpl"], b["vpl"]) == ("4", "2") and int(a["team"]) * 2 == int(b["team"]), (N, a, b)
    for N in (8192, 16384):
        assert parse(rn.norm_describe("add_rms", 64, N, "f32")) == parse(rn.norm_describe("rms", 64, N, "f32"))


@no_device_only
def test_fp8_validation():
    Q = 0x900000
    ok = lambda st: st not in (ALIAS, BAD_ARG, NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_EPS)
    assert rn.rms_fp8_fwd(X, G, Q, RSTD, 4, 64, 1e-6, 0.0, 2, None) == BAD_ARG        # scale 0
    assert rn.rms_fp8_fwd(X, G, Q, RSTD, 4, 64, 1e-6, -1.0, 2, None) == BAD_ARG
    assert rn.rms_fp8_fwd(X, G, Q, RSTD, 4, 64, 1e-6, float("inf"), 2, None) == BAD_ARG
    assert rn.rms_fp8_fwd(X, G, Q, RSTD, 4, 64, 1e-6, float("nan"), 2, None) == BAD_ARG
    assert rn.rms_fp8_fwd(X, G, Q, RSTD, 4, 64, 1e-6, 1e-45, 2, None) == BAD_ARG     # 1/scale overflows
    assert rn.rms_fp8_fwd(X, G, None, RSTD, 4, 64, 1e-6, 1.0, 2, None) == NULL_ARG
    assert rn.rms_fp8_fwd(X, G, X, RSTD, 4, 64, 1e-6, 1.0, 2, None) == ALIAS          # codes over x
    assert rn.rms_fp8_fwd(X, G, X + 128, RSTD, 4, 64, 1e-6, 1.0, 2, None) == ALIAS
    assert ok(rn.rms_fp8_fwd(X, G, X + 4 * 64 * 2, RSTD, 4, 64, 1e-6, 1.0, 2, None))  # right after x
    assert rn.rms_fp8_fwd(X, G, Q, Q + 200, 4, 64, 1e-6, 1.0, 2, None) == ALIAS       # rstd inside codes
    assert ok(rn.rms_fp8_fwd(X, G, Q, Q + 256, 4, 64, 1e-6, 1.0, 2, None))            # 4 x 64 bytes
    # with the residual add: the sum may go over the residual, the codes never over x
    assert ok(rn.add_rms_fp8_fwd(X, R, G, Q, R, RSTD, 4, 64, 1e-6, 0.5, 2, None))
    assert rn.add_rms_fp8_fwd(X, R, G, X, H, RSTD, 4, 64, 1e-6, 0.5, 2, None) == ALIAS
    assert rn.add_rms_fp8_fwd(X, None, G, Q, H, RSTD, 4, 64, 1e-6, 0.5, 2, None) == NULL_ARG
    assert ok(rn.rms_fp8_fwd(X, G, Q + 1, RSTD, 4, 64, 1e-6, 1.0, 2, None))          # codes: any byte address


def test_fp8_plans_like_rms():
    # FP8 output: the RMSNorm tiles up to 512 vectors a row and on split
    # rows (the residual add's tiles with it); 8 vectors per lane past 1024
    for N in (1024, 4096, 1 << 20):
        for op in ("rms_fp8", "add_rms_fp8"):
            assert parse(rn.norm_describe(op, 64, N, "bf16")) == parse(rn.norm_describe("rms", 64, N, "bf16"))
    for N in (8192, 16384):
        assert parse(rn.norm_describe("add_rms_fp8", 64, N, "bf16")) == parse(rn.norm_describe("add_rms", 64, N, "bf16"))
    assert parse(rn.norm_describe("rms_fp8", 64, 8192, "bf16")) == parse(rn.norm_describe("add_rms", 64, 8192, "bf16"))
    d = parse(rn.norm_describe("rms_fp8", 64, 16384, "bf16"))
    assert (d["team"], d["vpl"]) == ("256", "8"), d


def test_rms_rejects_beta_and_mean():
    assert rn.rms_fwd(X, G, B, Y, None, RSTD, 4, 64, 1e-6, 0, None) == BAD_ARG
    assert rn.rms_fwd(X, G, None, Y, MEAN, RSTD, 4, 64, 1e-6, 0, None) == BAD_ARG


def test_ln_mean_rstd_overlap_rejected():
    assert call("ln", mean=RSTD) == ALIAS
    assert call("ln", mean=RSTD - 8, M=4) == ALIAS      # [RSTD-8, RSTD+8) overlaps


def parse(desc):
    return dict(kv.split("=") for kv in desc.split())


@pytest.mark.parametrize("op,M,N,dtype,want", [
    ("ln", 128, 1024, "f32", dict(path="rows", team="128", vpl="2", epv="4")),
    ("rms", 8192, 4096, "f32", dict(path="rows", team="512", vpl="2", epv="4")),
    ("ln", 16384, 8192, "bf16", dict(path="rows", team="256", vpl="4", epv="8")),
    ("rms", 65536, 2048, "f32", dict(path="rows", team="32", vpl="16", epv="4", rows_per_wg="8")),
    ("rms", 65536, 2048, "bf16", dict(path="rows", team="64", vpl="4", epv="8")),
    ("ln", 4096, 5120, "bf16", dict(path="rows", team="64", vpl="10", epv="8")),
    ("ln", 64, 1 << 20, "bf16", dict(path="split", mode="two", chunks="64", apply_chunks="64", epv="8",
                                      batch_rows="64", grid="4096", apply_grid="4096")),
])
def test_plans_of_the_measured_configurations(op, M, N, dtype, want):
    d = parse(rn.norm_describe(op, M, N, dtype))
    for k, v in want.items():
        assert d[k] == v, (k, d)


def test_realigned_plans():
    """x alone off 16 bytes: the aligned plan's row tile on the realigned
    kernel, except RMSNorm fp32's 32 x 16 (slower realigned); split rows on
    the realigned two kernels; the residual add and N off whole vectors keep
    the element-wise plan."""
    def d(op, M, N, dtype, al):
        return parse(rn.norm_describe(op, M, N, dtype, aligned=al))
    for op, M, N, dtype in [("ln", 16384, 8192, "bf16"), ("rms", 65536, 2048, "bf16"), ("rms_fp8", 512, 4096, "f16"),
                            ("ln", 262144, 256, "bf16"), ("ln", 8192, 8192, "f32"), ("ln", 64, 65536, "bf16"),
                            ("ln", 4096, 5120, "bf16"), ("rms", 16384, 8192, "bf16")]:
        a, x = d(op, M, N, dtype, True), d(op, M, N, dtype, "x")
        assert x.pop("x") == "realigned" and x == a, (op, M, N, dtype, a, x)
    x = d("rms", 65536, 2048, "f32", "x")
    assert x["x"] == "realigned" and (x["team"], x["vpl"]) != ("32", "16"), x
    for op, N, dtype in [("ln", 1 << 20, "bf16"), ("rms", 1 << 20, "f32"), ("rms_fp8", 140000, "f16")]:
        x = d(op, 64, N, dtype, "x")
        assert x["path"] == "split" and x["mode"] == "two" and x["x"] == "realigned", x
        assert x["epv"] == str(16 // (4 if dtype == "f32" else 2)), x
    for op, N, dtype in [("add_rms", 4096, "bf16"), ("ln", 4100, "bf16"), ("add_rms", 1 << 20, "bf16")]:
        assert "x" not in d(op, 64, N, dtype, "x") and d(op, 64, N, dtype, "x") == d(op, 64, N, dtype, False)


@pytest.mark.parametrize("op,N,dtype,want", [
    ("ln", 16384, "bf16", ("rows", "256", "8")),
    ("ln", 32768, "bf16", ("rows", "512", "8")),
    ("ln", 65536, "bf16", ("rows", "1024", "8")),
    ("ln", 131072, "bf16", ("split", None, None)),
    ("ln", 8192, "f32", ("rows", "512", "4")),
    ("ln", 16384, "f32", ("rows", "512", "8")),
    ("ln", 32768, "f32", ("rows", "1024", "8")),
    ("ln", 65536, "f32", ("split", None, None)),
    ("rms", 16384, "bf16", ("rows", "1024", "2")),
    ("rms", 8192, "bf16", ("rows", "512", "2")),
    ("rms", 4096, "bf16", ("rows", "128", "4")),
    ("rms", 6144, "f16", ("rows", "512", "2")),
    ("add_rms", 8192, "bf16", ("rows", "256", "4")),
    ("rms_fp8", 8192, "bf16", ("rows", "256", "4")),
    ("rms_fp8", 12288, "bf16", ("rows", "256", "8")),
    ("rms_fp8", 32768, "bf16", ("rows", "512", "8")),
    ("rms_fp8", 8192, "f32", ("rows", "256", "8")),
    ("rms", 8192, "f32", ("rows", "1024", "2")),
    ("rms", 131072, "bf16", ("split", None, None)),
])
def test_long_row_tiles(op, N, dtype, want):
    d = parse(rn.norm_describe(op, 64, N, dtype))
    if want[0] == "split":
        assert d["path"] == "split", d
    else:
        assert (d["path"], d["team"], d["vpl"]) == want, d


def test_small_rows_share_a_wavefront():
    for N in (16, 64, 200, 256, 512, 1024):       # aligned bf16 rows of at most 2 KiB
        d = parse(rn.norm_describe("rms", 1000, N, "bf16"))
        assert int(d["team"]) <= 32 and int(d["rows_per_wg"]) >= 8, (N, d)
    for N in (16, 64, 256):                        # fp32 rows of at most 1 KiB
        d = parse(rn.norm_describe("ln", 1000, N, "f32"))
        assert int(d["team"]) <= 32, (N, d)


def test_unaligned_plans_take_the_elementwise_path():
    d = parse(rn.norm_describe("ln", 1, 10, "f32"))          # 40-byte rows
    assert d["epv"] == "1" and d["path"] == "rows"
    d = parse(rn.norm_describe("ln", 64, 4096, "bf16", aligned=False))
    assert d["epv"] == "1"


def test_one_wavefront_tiles_only_for_few_rows_that_fill_them():
    """64 lanes x 5 or 10 vectors when that covers a row of 16-byte vectors
    exactly and there are at most 4096 rows; the wider tiles otherwise."""
    for dtype, N, vpl in (("bf16", 5120, 10), ("f16", 5120, 10), ("bf16", 2560, 5), ("f32", 2560, 10),
                          ("f32", 1280, 5)):
        for op in ("ln", "rms", "add_rms", "rms_fp8", "add_rms_fp8"):
            d = parse(rn.norm_describe(op, 4096, N, dtype))
            assert (d["team"], d["vpl"], d["rows_per_wg"], d["grid"]) == ("64", str(vpl), "4", "1024"), (op, d)
        assert parse(rn.norm_describe("ln", 4097, N, dtype))["team"] != "64"
        assert parse(rn.norm_describe("ln", 4096, N, dtype, False))["epv"] == "1"
        assert parse(rn.norm_describe("ln", 4096, N, dtype, False))["vpl"] not in ("5", "10")
    for dtype, N in (("bf16", 5128), ("bf16", 4096), ("f32", 2048), ("bf16", 1280)):
        assert parse(rn.norm_describe("ln", 100, N, dtype))["vpl"] not in ("5", "10")


def test_every_row_fits_its_tile():
    for dtype, e in (("f32", 4), ("bf16", 2), ("f16", 2)):
        for N in list(range(1, 70)) + [127, 1000, 1023, 1025, 5120, 8191, 8193, 65536, 131072, 131073, 1 << 20]:
            for aligned in (True, False):
                d = parse(rn.norm_describe("ln", 3, N, dtype, aligned))
                epv = int(d["epv"])
                if aligned and (N * e) % 16 == 0:
                    assert epv == 16 // e
                else:
                    assert epv == 1
                nv = N // epv
                if d["path"] == "rows":
                    assert int(d["team"]) * int(d["vpl"]) >= nv
                else:
                    assert int(d["chunks"]) * int(d["wg"]) * int(d["vpl"]) >= nv
                    assert int(d["apply_chunks"]) * int(d["apply_wg"]) * int(d["apply_vpl"]) >= nv


def test_split_rows_run_in_batches_of_about_256_mib():
    d = parse(rn.norm_describe("ln", 4096, 1 << 18, "bf16"))      # 512 KiB rows: 512 per batch
    assert (d["mode"], d["batch_rows"], d["chunks"]) == ("two", "512", "16")
    assert int(d["grid"]) == 512 * 16 and int(d["apply_grid"]) == 512 * int(d["apply_chunks"])
    d = parse(rn.norm_describe("rms", 5, 1 << 24, "f32"))          # 64 MiB rows: 4 per batch
    assert d["batch_rows"] == "4" and int(d["chunks"]) * 8192 == 1 << 24
    d = parse(rn.norm_describe("ln", 1, 200000, "f16", aligned=False))
    assert (d["batch_rows"], d["epv"], d["chunks"]) == ("1", "1", str(-(-200000 // 2048)))


def test_split_batch_override(monkeypatch):
    monkeypatch.setenv("MI355NORM_SPLIT_BATCH", str(3 * 140000 * 2))
    d = parse(rn.norm_describe("ln", 7, 140000, "bf16"))
    assert d["batch_rows"] == "3" and int(d["work"]) == 3 * int(d["chunks"])
    monkeypatch.setenv("MI355NORM_SPLIT_BATCH", "1")               # below one row: one row per batch
    assert parse(rn.norm_describe("ln", 7, 140000, "bf16"))["batch_rows"] == "1"


def test_overrides(monkeypatch):
    monkeypatch.setenv("MI355NORM_PATH", "split")
    assert parse(rn.norm_describe("ln", 64, 8192, "bf16"))["path"] == "split"
    monkeypatch.setenv("MI355NORM_PATH", "split2")
    assert parse(rn.norm_describe("ln", 64, 8192, "bf16"))["mode"] == "two"
    monkeypatch.setenv("MI355NORM_PATH", "rows")
    with pytest.raises(RuntimeError):
        rn.norm_describe("ln", 64, 1 << 20, "bf16")     # does not fit one workgroup
    monkeypatch.delenv("MI355NORM_PATH")
    monkeypatch.setenv("MI355NORM_TILE", "64x16")
    d = parse(rn.norm_describe("ln", 64, 8192, "bf16"))
    assert (d["team"], d["vpl"]) == ("64", "16")
    monkeypatch.setenv("MI355NORM_TILE", "64x2")         # too small for the row
    with pytest.raises(RuntimeError):
        rn.norm_describe("ln", 64, 8192, "bf16")
    monkeypatch.delenv("MI355NORM_TILE")
    monkeypatch.setenv("MI355NORM_GRID", "1024")
    assert parse(rn.norm_describe("ln", 16384, 8192, "bf16"))["grid"] == "1024"


# ---------------------------------------------------------------------------
# norm_fwd: row strides
# ---------------------------------------------------------------------------

def strided(op="ln", M=4, N=64, dtype=0, **kw):
    args = dict(x=X, y=Y, gamma=G, rstd=RSTD, eps=1e-5, scale=1.0)
    if op == "ln":
        args.update(beta=B, mean=MEAN)
    if op.startswith("add"):
        args.update(residual=R, residual_out=H)
    args.update(kw)
    x, y = args.pop("x"), args.pop("y")
    return rn.norm_fwd(op, dtype, M, N, x, y, **args)


def passes(st):
    return st not in (ALIAS, BAD_ARG, NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_EPS)


@pytest.mark.parametrize("cls,cname", [(rn.NormArgs, "norm_args"), (rn.NormBwdArgs, "norm_bwd_args")])
def test_args_structs_match_the_header(tmp_path, cls, cname):
    import subprocess
    fields = [f[0] for f in cls._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mi355norm.h"\nint main(void){\n'
                   f'printf("%zu", sizeof({cname}));\n'
                   + "".join(f'printf(" %zu", offsetof({cname}, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(os.path.dirname(HEADER)), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(cls)] + [getattr(cls, f).offset for f in fields]
    assert got == want


@no_device_only
def test_strides_are_validated():
    assert strided(ld_x=63) == BAD_SHAPE                 # shorter than a row
    assert strided(ld_y=1) == BAD_SHAPE
    assert strided(op="add_rms", ld_residual=10) == BAD_SHAPE
    assert strided(ld_x=1 << 62) == BAD_SHAPE            # the matrix would not fit 2^63 bytes
    assert passes(strided(ld_x=0, ld_y=0))               # 0 means N
    assert passes(strided(ld_x=100, ld_y=64))
    assert rn.norm_fwd("ln", 0, 4, 64, X, None) == NULL_ARG
    assert rn.norm_fwd(7, 0, 4, 64, X, Y) == BAD_ARG


@no_device_only
def test_strided_overlaps_are_exact_for_one_shared_stride():
    # x and y interleaved in one [M, 2N] fp32 buffer: no common byte
    assert passes(strided(x=X, y=X + 64 * 4, ld_x=128, ld_y=128, M=8))
    assert strided(x=X, y=X + 32 * 4, ld_x=128, ld_y=128, M=8) == ALIAS      # half a row over
    assert strided(x=X, y=X + 127 * 4, ld_x=128, ld_y=128, M=8) == ALIAS     # last row's tail
    assert passes(strided(x=X + 64 * 4, y=X, ld_x=128, ld_y=128, M=8))
    # a vector in the gap between rows of y is fine, on a row it is not
    assert passes(strided(y=Y, ld_y=128, M=8, gamma=Y + 64 * 4, beta=None))
    assert strided(y=Y, ld_y=128, M=8, gamma=Y + 256 * 4, beta=None) == ALIAS
    # different strides with intersecting spans: rejected (not resolved exactly)
    assert strided(x=X, y=X + 64 * 4, ld_x=128, ld_y=192, M=8) == ALIAS


@no_device_only
def test_strided_in_place_residual_needs_the_same_stride():
    assert passes(strided(op="add_rms", residual=R, residual_out=R, ld_residual=80, ld_residual_out=80))
    assert strided(op="add_rms", residual=R, residual_out=R, ld_residual=80, ld_residual_out=96) == ALIAS
    assert passes(strided(op="add_rms", x=X, y=X, ld_x=72, ld_y=72))


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

A = 1 << 20   # fake, 16-byte aligned "device" addresses: validation rejects before any use


def ln_bwd(dy=A, x=2 * A, gamma=None, mean=3 * A, rstd=4 * A, dx=5 * A, dgamma=None, dbeta=None, M=4, N=64,
           dtype=rn.NORM_BF16):
    return rn.ln_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, M, N, dtype, None)


def rms_bwd(dy=A, x=2 * A, gamma=None, rstd=4 * A, dx=5 * A, dgamma=None, M=4, N=64, dtype=rn.NORM_BF16):
    return rn.rms_bwd(dy, x, gamma, rstd, dx, dgamma, M, N, dtype, None)


def test_bwd_validation():
    assert ln_bwd(dtype=7) == BAD_DTYPE
    assert ln_bwd(M=-1) == BAD_SHAPE
    assert ln_bwd(N=0) == BAD_SHAPE
    assert ln_bwd(N=(1 << 24) + 1) == BAD_SHAPE
    assert ln_bwd(dy=None) == NULL_ARG
    assert ln_bwd(x=None) == NULL_ARG
    assert ln_bwd(dx=None) == NULL_ARG
    assert ln_bwd(mean=None) == NULL_ARG               # LayerNorm needs the mean
    assert ln_bwd(rstd=None) == NULL_ARG
    assert rms_bwd(rstd=None) == NULL_ARG
    assert ln_bwd(dy=A + 1) == BAD_ARG                 # misaligned for bf16
    assert ln_bwd(mean=3 * A + 2) == BAD_ARG
    assert ln_bwd(dgamma=6 * A + 2) == BAD_ARG
    # outputs overlapping inputs or each other
    assert ln_bwd(dx=A + 64) == ALIAS                  # dx inside dy, shifted
    assert ln_bwd(dgamma=A) == ALIAS
    assert ln_bwd(dgamma=6 * A, dbeta=6 * A + 128) == ALIAS
    assert ln_bwd(dbeta=3 * A) == ALIAS                # over mean
    assert rms_bwd(dgamma=4 * A) == ALIAS              # over rstd


def test_bwd_exact_in_place_passes_validation():
    # dx exactly over dy or over x is allowed; with M = 0 nothing launches
    assert ln_bwd(dx=A, M=0) == OK
    assert ln_bwd(dx=A, dy=None, M=4) == NULL_ARG
    assert rms_bwd(dx=2 * A, M=0) == OK


def test_bwd_empty_needs_no_pointers():
    assert ln_bwd(dy=None, x=None, mean=None, rstd=None, dx=None, M=0) == OK
    assert rms_bwd(dy=None, x=None, rstd=None, dx=None, M=0) == OK


@pytest.mark.parametrize("N,dtype,aligned,ln_rows,rms_rows", [
    (32768, "bf16", True, True, True), (32776, "bf16", True, False, False),
    (16384, "f32", True, True, True), (24576, "f32", True, True, False), (16416, "f32", True, True, False),
    (24608, "f32", True, False, False), (32768, "f32", True, False, False),
    (16384, "bf16", False, True, True), (16385, "f16", False, False, False), (16384, "f32", False, True, True),
    (1, "f32", False, True, True), (1 << 24, "bf16", True, False, False)])
def test_bwd_row_kernel_limit_then_split(N, dtype, aligned, ln_rows, rms_rows):
    # the row kernel up to 32768 elements (16384 unaligned); fp32 rows that
    # need 32 elements per lane go split (LayerNorm only past 24576)
    for op, rows in (("ln", ln_rows), ("rms", rms_rows)):
        want = "path=bwd " if rows else "path=bwd_split "
        assert rn.norm_bwd_describe(op, 1024, N, dtype, aligned).startswith(want), (op, N, dtype)
    with pytest.raises(RuntimeError, match="bad shape"):
        rn.norm_bwd_describe("ln", 1024, (1 << 24) + 1, dtype, aligned)


def test_bwd_split_plans():
    d = dict(kv.split("=") for kv in rn.norm_bwd_describe("ln", 64, 1 << 20, "bf16", True).split())
    # chunk sums over 256 x 2 vectors, dx over 256 x 2, about two workgroups per CU (256 here)
    assert d["chunks"] == "256" and d["apply_chunks"] == "256" and d["apply_vpl"] == "2" and d["sums_vpl"] == "2"
    assert d["batch_rows"] == "64" and d["partial_rows"] == "2" and d["apply_grid"] == "512"
    d = dict(kv.split("=") for kv in rn.norm_bwd_describe("rms", 100000, 40000, "f32", True).split())
    # every row in one batch
    assert int(d["batch_rows"]) == 100000
    assert int(d["partial_rows"]) == -(-512 // int(d["apply_chunks"]))
    d = dict(kv.split("=") for kv in rn.norm_bwd_describe("ln", 3, 1 << 24, "f16", False).split())
    assert d["epv"] == "1" and int(d["partial_rows"]) == 1 and d["batch_rows"] == "3"


def _bwd_plan(op, M, N, dtype, aligned=True):
    d = dict(kv.split("=") for kv in rn.norm_bwd_describe(op, M, N, dtype, aligned).split())
    return {k: (v if k in ("path", "op", "mode") else int(v)) for k, v in d.items()}


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("aligned", [True, False])
def test_bwd_every_row_fits_its_tile(dtype, aligned):
    e = 4 if dtype == "f32" else 2
    limit = 32768 if aligned else 16384
    for N in [1, 7, 8, 64, 100, 768, 1000, 1024, 4096, 5120, 8192, 12288, 16384, 24576, 32768]:
        if N > limit or (aligned and (N * e) % 16):
            continue
        p = _bwd_plan("ln", 4096, N, dtype, aligned)
        if p["path"] == "bwd_split":
            assert dtype == "f32" and aligned and N > 24576
            continue
        epv = p["epv"]
        assert epv == (16 // e if aligned else 1)
        slots = p["team"] * p["vpl"] * epv
        assert slots >= N and (p["team"] == 8 or N >= slots // 4)
        assert p["vpl"] * epv <= 32 and 8 <= p["team"] <= 1024
        assert p["wg"] == 1024 and p["rows_per_wg"] == 1024 // p["team"]
        assert p["grid"] == min(p["work"], 256) == p["partial_rows"]      # one workgroup per CU
        if aligned and p["team"] * epv < N:
            assert p["team"] == 1024                    # more than one vector per lane only past 1024 lanes


def test_bwd_split_on_request(monkeypatch):
    monkeypatch.setenv("MI355NORM_PATH", "split")
    assert rn.norm_bwd_describe("ln", 4096, 8192, "bf16").startswith("path=bwd_split ")
    monkeypatch.setenv("MI355NORM_SPLIT_BATCH", str(1 << 20))
    d = dict(kv.split("=") for kv in rn.norm_bwd_describe("ln", 4096, 8192, "bf16").split())
    assert d["batch_rows"] == str((1 << 20) // (2 * 8192 * 2))


def test_bwd_grid_override(monkeypatch):
    monkeypatch.setenv("MI355NORM_GRID", "100")
    assert _bwd_plan("rms", 16384, 8192, "bf16")["grid"] == 100
    monkeypatch.setenv("MI355NORM_TILE", "256x4")
    p = _bwd_plan("rms", 16384, 8192, "bf16")
    assert (p["team"], p["vpl"]) == (256, 4)
    monkeypatch.setenv("MI355NORM_TILE", "128x4")        # too small for the row
    with pytest.raises(RuntimeError):
        rn.norm_bwd_describe("rms", 16384, 8192, "bf16")
    monkeypatch.setenv("MI355NORM_TILE", "1024x8")       # 64 bf16 elements per lane: not instantiated
    with pytest.raises(RuntimeError):
        rn.norm_bwd_describe("rms", 16384, 8192, "bf16")


def nbwd(op="ln", dy=A, x=2 * A, dx=5 * A, mean=3 * A, rstd=4 * A, M=4, N=64, **kw):
    return rn.norm_bwd(op, "bf16", M, N, dy, x, dx, mean=mean if op == "ln" else kw.pop("mean_rms", None),
                       rstd=rstd, **kw)


def test_bwd_strides_are_validated():
    assert rn._lib.norm_bwd(None, None) == NULL_ARG
    assert nbwd(ld_dy=63) == BAD_SHAPE                       # stride below N
    assert nbwd(ld_dx=1 << 62) == BAD_SHAPE                  # matrix beyond 2^63 bytes
    assert nbwd(op=7) == BAD_ARG
    assert nbwd(op="add_rms") == BAD_ARG
    assert nbwd(op="rms", mean_rms=3 * A) == BAD_ARG         # RMSNorm takes no mean
    assert nbwd(M=0, dy=None, x=None, dx=None, mean=None, rstd=None) == OK
    # interleaved rows of dy and dx share no byte: accepted (nothing launches at M = 0)
    assert nbwd(M=0, ld_dy=128, ld_dx=128, dx=A + 128) == OK
    # dx over dy with another stride: rejected; with the same pointer and stride: accepted
    assert nbwd(ld_dy=128, ld_dx=64, dx=A) == ALIAS
    assert nbwd(ld_dy=128, ld_dx=128, dx=A, M=0) == OK
    # rows of dx running into x
    assert nbwd(ld_dx=64, dx=2 * A - 64 * 2 * 2) == ALIAS


def test_bwd_strided_plans_need_aligned_rows():
    assert "epv=8" in rn.norm_bwd_describe("ln", 64, 1024, "bf16", True)
    assert "epv=1" in rn.norm_bwd_describe("ln", 64, 1024, "bf16", False)


def test_noalloc_validates_and_refuses_on_the_host(monkeypatch):
    """norm_fwd_noalloc: the same validation as norm_fwd, and the refusals of
    what its fixed scratch cannot hold, all before any HIP call."""
    assert rn._lib.norm_fwd_noalloc(None, None) == NULL_ARG
    fake = 1 << 40   # never dereferenced: every case below returns before a launch
    assert rn.norm_fwd_noalloc("ln", "bf16", 0, 1024, None, None) == OK
    assert rn.norm_fwd_noalloc("ln", 7, 4, 1024, fake, fake + (1 << 30)) == BAD_DTYPE
    assert rn.norm_fwd_noalloc("ln", "bf16", 4, 1024, fake, fake + 1024) == ALIAS
    # a forced split of 2^20 short rows needs 8 MiB of partials in one batch
    monkeypatch.setenv("MI355NORM_PATH", "split")
    assert rn.norm_fwd_noalloc("rms", "f32", 1 << 20, 64, fake, fake + (1 << 30), eps=1e-6) == 8
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    assert rn.norm_fwd_noalloc("rms", "f32", 40, 100000, fake, fake + (1 << 30), eps=1e-6) == BAD_ARG


@pytest.mark.parametrize("dtype,N,aligned", [("bf16", 16385, False), ("f32", 16385, False), ("bf16", 65544, True),
                                             ("f32", 32772, True), ("bf16", 1 << 20, True), ("f16", 1 << 24, True)])
def test_noalloc_scratch_holds_every_default_split_batch(dtype, N, aligned):
    """The largest partials of the default two-kernel schedule (rows of one
    batch x chunks per row x 8 bytes) fit the 1 MiB scratch: the worst case is
    the shortest split rows of a 2-byte type on the element-wise path."""
    d = dict(kv.split("=") for kv in rn.norm_describe("ln", 1 << 30, N, dtype, aligned=aligned).split())
    assert d["path"] == "split" and d["mode"] == "two"
    assert int(d["batch_rows"]) * int(d["chunks"]) * 8 <= 1 << 20


def test_cpython_calls_match_ctypes():
    """The CPython module of the per-call entry points is built and bound,
    and returns what the ctypes call of the same library function returns
    for every validation outcome (no device is touched: each case fails
    before any launch, or has M == 0)."""
    assert rn._calls is not None and rn.ln_fwd is rn._calls.ln_fwd
    P, Q, S = 0x100000, 0x200000, 0x300000          # 16-byte aligned, disjoint for small shapes
    cases = {
        "ln_fwd": [(P, None, None, S, None, None, 0, 64, 1e-5, 2, None),                  # M = 0
                   (P, None, None, S, None, None, 4, 64, 1e-5, 9, None),                  # dtype
                   (P, None, None, S, None, None, 4, 0, 1e-5, 2, None),                   # N
                   (P, None, None, S, None, None, 4, 64, -1.0, 2, None),                  # eps
                   (None, None, None, S, None, None, 4, 64, 1e-5, 2, None),               # null x
                   (P + 1, None, None, S, None, None, 4, 64, 1e-5, 2, None),              # misaligned
                   (P, None, None, P + 64, None, None, 4, 64, 1e-5, 2, None)],            # alias
        "rms_fwd": [(P, None, Q, S, None, None, 4, 64, 1e-6, 2, None),                  # beta given
                    (P, None, None, S, None, None, -1, 64, 1e-6, 0, None)],
        "add_rms_fwd": [(P, None, None, S, None, None, 4, 64, 1e-6, 2, None),           # null residual
                        (P, Q, None, S, Q, None, 0, 64, 1e-6, 2, None)],
        "rms_fp8_fwd": [(P, None, S, None, 4, 64, 1e-6, 0.0, 2, None),                  # scale
                        (P, None, S, None, 0, 64, 1e-6, 1.0, 2, None)],
        "add_rms_fp8_fwd": [(P, None, None, S, Q, None, 4, 64, 1e-6, 1.0, 2, None),
                            (P, Q, None, S, None, None, 4, 64, 1e-6, 1.0, 1, None)],
        "ln_bwd": [(P, Q, None, None, None, S, None, None, 4, 64, 2, None),             # null statistics
                   (P, Q, None, S, S + 64, None, None, None, 0, 64, 2, None)],
        "rms_bwd": [(P, Q, None, None, S, None, 4, 64, 2, None),
                    (P, Q, None, S, S + 64, None, 4, 64, 7, None)],
    }
    for name, calls in cases.items():
        for args in calls:
            got = getattr(rn._calls, name)(*args)
            want = getattr(rn._lib, name)(*args)
            assert got == want, (name, args, got, want)
    with pytest.raises(TypeError):
        rn._calls.ln_fwd(P, None, None, S, None, None, 4, 64, 1e-5, 2)             # one argument short
    with pytest.raises(TypeError):
        rn._calls.rms_fwd("x", None, None, S, None, None, 4, 64, 1e-6, 2, None)     # not an address
    with pytest.raises(OverflowError):
        rn._calls.ln_fwd(P, None, None, S, None, None, 0, 64, 1e-5, 2 ** 32 + 2, None)   # would wrap to bf16
