"""The C ABI from plain C: tests/c_abi/abi_example.c (gcc, the HIP runtime's
C API, no Python or torch in the caller) links libmi355norm.so, runs ln_fwd,
rms_fwd and ln_bwd on the device and writes its results; the GPU test checks
them against the oracle."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import oracle  # noqa: E402
import rmsnorm_forward_amd as rn  # noqa: E402
import workloads  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_example.c")


def compile_example(out_dir) -> str:
    exe = os.path.join(str(out_dir), "abi_example")
    libdir = os.path.dirname(rn.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", SRC,
                    "-L", libdir, "-lmi355norm", "-L", "/opt/rocm/lib", "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    return exe


def test_plain_c_caller_compiles_and_links(tmp_path):
    exe = compile_example(tmp_path)
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
def test_plain_c_caller_matches_the_oracle(tmp_path):
    M, N = 37, 1000
    d = workloads.gen_ln_normal(91, M, N, "f32", loc=2.0, scale=1.5)
    dy = workloads.normal(np.random.default_rng(92), (M, N), 0.0, 1.0)
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(np.array([M, N], np.int64).tobytes())
        for a in (d["x"], d["gamma"], d["beta"], dy):
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
    exe = compile_example(tmp_path)
    out = tmp_path / "out.bin"
    print("[c-abi] running the plain C caller", flush=True)
    r = subprocess.run([exe, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    v = np.fromfile(out, np.float32)
    sizes = [M * N, M, M, M * N, M, M * N, N, N]
    assert v.size == sum(sizes)
    y_ln, mean, rstd, y_rms, rstd_rms, dx, dg, db = np.split(v, np.cumsum(sizes)[:-1])
    yr, mr, rr = oracle.ln_fwd(d["x"], d["gamma"], d["beta"], "f32", 1e-5)
    assert np.max(np.abs(y_ln.reshape(M, N) - yr)) <= 2e-5
    assert np.max(np.abs(rstd - rr) / rr) <= 1e-5
    var = 1.0 / rr ** 2
    assert np.max(np.abs(mean - mr) / np.maximum(np.abs(mr), np.sqrt(var))) <= 1e-5
    yr2, rr2 = oracle.rms_fwd(d["x"], d["gamma"], "f32", 1e-6)
    assert np.max(np.abs(y_rms.reshape(M, N) - yr2)) <= 2e-5
    assert np.max(np.abs(rstd_rms - rr2) / rr2) <= 1e-5
    # the backward ran on the library forward's statistics; the oracle gets
    # its own (fp32), so the bar allows for their <= 1e-5 relative difference
    dxr, dgr, dbr = oracle.ln_bwd(dy, d["x"], d["gamma"], "f32", mr.astype(np.float32), rr.astype(np.float32))
    assert np.max(np.abs(dx.reshape(M, N) - dxr)) <= 1e-4 * np.abs(dxr).max()
    assert np.max(np.abs(dg - dgr)) <= 1e-4 * np.abs(dgr).max()
    assert np.max(np.abs(db - dbr)) <= 1e-5 * np.abs(dy).sum(0).max()
