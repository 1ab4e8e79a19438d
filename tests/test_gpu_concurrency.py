"""Host threads calling the library at once, each on its own stream: the
split-row forward and the backward, row kernel and split rows (which keep
workspaces per device and stream), give the same bits as the same calls made
one after another.  The RMSNorm job takes the single pass on rows of 2^20,
with teams sized for the whole GPU: four such launches at once cannot all be
resident, so workgroups whose teammates start late reach the end of their
bounded wait and recompute the row, which must not change a bit."""
from __future__ import annotations

import threading

import numpy as np
import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
gpu_runner = pytest.importorskip("gpu_runner")
rn = pytest.importorskip("rmsnorm_forward_amd")


def job(k):
    """Inputs of thread k: a split-path LayerNorm (rows of 300000), a
    LayerNorm backward (512 x 4096) and a split-row LayerNorm backward
    (3 x 70000), bf16."""
    f = workloads.gen_ln_normal(200 + k, 4, 300000, "bf16")
    b = workloads.gen_bwd(300 + k, 512, 4096, "bf16", "ln_bwd")
    s = workloads.gen_bwd(400 + k, 3, 70000, "bf16", "ln_bwd")
    r = workloads.gen_rms_uniform(500 + k, 16, 1 << 20, "bf16")
    dev = lambda a: gpu_runner.to_device(a, "bf16")
    return {"x": dev(f["x"]).view(4, 300000), "g": dev(f["gamma"]), "b": dev(f["beta"]),
            "rx": dev(r["x"]).view(16, 1 << 20), "rg": dev(r["gamma"]),
            "bx": dev(b["x"]).view(512, 4096), "bg": dev(b["gamma"]), "dy": dev(b["dy"]).view(512, 4096),
            "sx": dev(s["x"]).view(3, 70000), "sg": dev(s["gamma"]), "sdy": dev(s["dy"]).view(3, 70000)}


def run_job(t, stream):
    with torch.cuda.stream(stream):
        y, mean, rstd = rn.layer_norm(t["x"], t["g"], t["b"], 1e-5)
        _, bm, br = rn.layer_norm(t["bx"], t["bg"], None, 1e-5)
        dx, dg, db = rn.layer_norm_backward(t["dy"], t["bx"], bm, br, t["bg"])
        _, sm, sr = rn.layer_norm(t["sx"], t["sg"], None, 1e-5)
        sdx, sdg, sdb = rn.layer_norm_backward(t["sdy"], t["sx"], sm, sr, t["sg"])
        ry, rr = rn.rms_norm(t["rx"], t["rg"], 1e-6)
    return [y, mean, rstd, dx, dg, db, sdx, sdg, sdb, ry, rr]


def bits(ts):
    return [a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32) for a in ts]


def test_threads_on_their_own_streams_match_serial_calls():
    plan = dict(kv.split("=") for kv in rn.norm_describe("rms", 16, 1 << 20, "bf16").split())
    assert plan["mode"] == "pass", plan
    jobs = [job(k) for k in range(4)]
    serial = [[a.clone() for a in run_job(t, torch.cuda.current_stream())] for t in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in jobs]
    results = [None] * len(jobs)
    errors = []

    def worker(k):
        try:
            out = None
            for _ in range(10):
                out = run_job(jobs[k], streams[k])
            streams[k].synchronize()
            results[k] = out
        except Exception as e:   # reported below, on the main thread
            errors.append(e)

    print("[gpu] 4 host threads, 4 streams", flush=True)
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for k in range(len(jobs)):
        for a, b in zip(bits(results[k]), bits(serial[k])):
            assert torch.equal(a, b), f"thread {k} differs from the serial result"
