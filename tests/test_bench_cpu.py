"""bench.py host logic that runs without a GPU: the one-GPU guard, the
counter-summary lookup, and the CPU baseline's byte accounting."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


def test_traffic_needs_matching_sources_and_plan(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k__w_counters.txt").write_text(
        "kernel_source_sha256: abc\nplan: path=rows team=256\ntraffic_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda kernel="norm_rows_kernel": "abc")
    assert bench.read_traffic("k", "w", "path=rows team=256") == 123.0
    assert bench.read_traffic("k", "w", "path=rows team=512") is None      # another tile
    assert bench.read_traffic("k", "other", "path=rows team=256") is None  # no summary
    monkeypatch.setattr(bench, "kernel_source_digest", lambda kernel="norm_rows_kernel": "def")
    assert bench.read_traffic("k", "w", "path=rows team=256") is None      # kernels changed


def test_kernel_digest_covers_the_device_code():
    for kernel, names in bench.KERNEL_SOURCES.items():
        for name in names:
            assert os.path.exists(os.path.join(ROOT, "rmsnorm_forward_amd", "csrc", name)), name
        assert len(bench.kernel_source_digest(kernel)) == 64
    # every kernel header is covered by some digest; the backward's own header
    # does not move the forward's digest
    covered = {n for names in bench.KERNEL_SOURCES.values() for n in names}
    headers = {f for f in os.listdir(os.path.join(ROOT, "rmsnorm_forward_amd", "csrc")) if f.endswith(".hpp")}
    assert headers - covered <= {"dispatch.hpp"}
    assert "backward.hpp" not in bench.KERNEL_SOURCES["norm_rows_kernel"]


def test_cpu_baseline_counts_the_rows_it_ran():
    w = workloads.Workload("t", "ln", "f32", 64, 256, 1e-5, 0, "")
    rng = np.random.default_rng(0)
    inp = {"x": rng.standard_normal((64, 256)).astype(np.float32),
           "gamma": np.ones(256, np.float32), "beta": np.zeros(256, np.float32)}
    cb = bench.cpu_baseline(w, inp, seconds=5.0)
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["unit"] == "GB/s"
    assert cb["sample"].startswith("64 of 64 rows") and cb["value"] > 0
    mt = bench.cpu_baseline(w, inp, seconds=5.0, threads=4)
    assert mt["cores"] == 4 and mt["sample"].startswith("64 of 64 rows") and "4 threads" in mt["sample"]


def test_cpu_baseline_of_the_backward():
    w = workloads.Workload("t", "ln_bwd", "bf16", 32, 512, 1e-5, 0, "")
    inp = workloads.gen_bwd(0, 32, 512, "bf16", "ln_bwd")
    cb = bench.cpu_baseline(w, inp, seconds=5.0)
    assert cb["sample"].startswith("32 of 32 rows") and "oracle.ln_bwd" in cb["sample"] and cb["value"] > 0
    assert w.ideal_bytes() == 3 * 32 * 512 * 2 + 512 * 2 + 512 * 8 + 32 * 8


def test_launches_per_step_follow_the_plan(monkeypatch):
    """Launch counts of one call, read from the library's own plan strings."""
    import rmsnorm_forward_amd as rn
    N = 1 << 20
    assert bench.launches_per_step(rn.norm_describe("ln", 16384, 8192, "bf16"), 16384) == 1
    assert bench.launches_per_step(rn.norm_describe("ln", 64, N, "bf16"), 64) == 2
    monkeypatch.setenv("MI355NORM_PATH", "splitpass")
    try:
        one = rn.norm_describe("ln", 64, N, "bf16")
    except RuntimeError:          # no device here: the single pass cannot be planned
        one = None
    if one is not None:
        assert bench.launches_per_step(one, 64) == 1
    # plan strings as the library writes them for the single passes
    fwd_pass = ("path=split mode=pass wg=512 vpl=8 epv=8 chunks=32 apply_wg=0 apply_vpl=0 apply_chunks=0 "
                "teams=16 batch_rows=64 grid=512 apply_grid=0 work=2048 workspace=32768")
    assert bench.launches_per_step(fwd_pass, 64) == 1
    bwd_pass = ("path=bwd_split mode=pass op=ln wg=1024 sums_vpl=2 apply_vpl=2 epv=8 chunks=64 apply_chunks=0 "
                "batch_rows=64 grid=256 apply_grid=0 partial_rows=4")
    assert bench.launches_per_step(bwd_pass, 64) == 2           # the pass, then the column sums
    monkeypatch.delenv("MI355NORM_PATH")
    monkeypatch.setenv("MI355NORM_SPLIT_BATCH", str(3 * N * 2))   # forward: 3 rows of x per batch
    assert bench.launches_per_step(rn.norm_describe("ln", 7, N, "bf16"), 7) == 6
    assert bench.launches_per_step(rn.norm_bwd_describe("ln", 16384, 8192, "bf16"), 16384) == 2
    monkeypatch.setenv("MI355NORM_SPLIT_BATCH", str(3 * 2 * N * 2))   # backward: 3 rows of dy and x
    p = rn.norm_bwd_describe("ln", 64, N, "bf16")
    assert "batch_rows=3" in p and "partial_rows=2" in p
    assert bench.launches_per_step(p, 64) == 3 * 22 + 1       # sums, row sums, apply per batch; column sums
    monkeypatch.delenv("MI355NORM_SPLIT_BATCH")
    assert bench.launches_per_step(rn.norm_bwd_describe("ln", 64, N, "bf16"), 64) == 4
    p = rn.norm_bwd_describe("rms", 8, 1 << 24, "bf16")
    assert "partial_rows=1" in p and bench.launches_per_step(p, 8) == 3   # one row group: no column sums


def test_source_digest_ignores_comments_only():
    """A change to comments or blank lines leaves the digest (and so the
    committed counter measurements) valid; a change to code does not."""
    a = "int f(int x) {  // one\n    return x + 1;\n}\n"
    b = "/* header\n   text */\nint f(int x) {\n\n    return x + 1;   // two\n}\n"
    c = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b) != bench._code_only(c)


def test_ceiling_streams_refuse_buffers_smaller_than_x_before_any_launch():
    """The ceiling streams copy x's bytes; y of FP8 codes is a quarter (bf16: a
    half) of them, so handing it over must fail on the host, before a launch."""
    import torch
    x = [torch.empty(4096, dtype=torch.bfloat16) for _ in range(2)]
    nbytes = x[0].numel() * x[0].element_size()
    y_fp8 = [torch.empty(4096, dtype=torch.uint8) for _ in range(2)]
    launched = []

    class Lib:
        def bench_stream(self, *a):
            launched.append(a)
            return 0

    try:
        bench.stream_ceilings(Lib(), x, y_fp8, nbytes, None, 1)
    except ValueError as e:
        assert "smaller" in str(e)
    else:
        raise AssertionError("FP8-sized destinations were accepted")
    assert not launched
    bench.check_stream_buffers(x, [torch.empty_like(t) for t in x], nbytes)   # x-sized: accepted


def test_matched_ceiling_refuses_short_buffers_before_any_launch():
    """The copies with a kernel's own streams check every source and every
    destination they write (kind 0: two; kind 1: one) before a launch."""
    import torch
    x = [torch.empty(4096, dtype=torch.bfloat16) for _ in range(2)]
    nbytes = x[0].numel() * x[0].element_size()
    short = [torch.empty(2048, dtype=torch.bfloat16) for _ in range(2)]
    launched = []

    class Lib:
        def bench_stream2(self, *a):
            launched.append(a)
            return 0

    for kind, s0, s1, d0, d1 in [(0, x, x, x, short), (0, x, short, x, x), (1, x, x, short, None),
                                 (1, short, x, x, None)]:
        try:
            bench.matched_ceiling(Lib(), kind, s0, s1, d0, d1, nbytes, None, 1)
        except ValueError as e:
            assert "smaller" in str(e)
        else:
            raise AssertionError(f"kind {kind}: a short buffer was accepted")
    assert not launched


def test_cpu_baseline_reports_the_median_of_three_passes_and_the_cpu():
    w = workloads.Workload("t", "rms", "f32", 32, 512, 1e-6, 0, "")
    rng = np.random.default_rng(1)
    inp = {"x": rng.standard_normal((32, 512)).astype(np.float32), "gamma": np.ones(512, np.float32)}
    cb = bench.cpu_baseline(w, inp, seconds=3.0)
    assert cb["runs"] == 3 and len(cb["run_seconds"]) == 3
    assert cb["cpu_model"] and "median of 3 passes" in cb["sample"]
    assert 1 <= bench.host_cores() <= 16
