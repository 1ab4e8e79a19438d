"""Calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The row path needs no workspace; the split paths and the backward use the
per-(device, stream) workspace, which exists once a call has run on the
capturing stream, so after a warm-up call there a capture records kernel
launches only (no allocation, no memset nodes).  Every replay, with eager
work and synchronisations between replays, must give the eager bits."""
from __future__ import annotations

import pytest

import __graft_entry__

__graft_entry__.ensure_built()

import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
gpu_runner = pytest.importorskip("gpu_runner")
rn = pytest.importorskip("rmsnorm_forward_amd")


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_capture_and_replay_forward_split_and_backward():
    """Forward rows, split forward, row-kernel backward and split backward."""
    dev = lambda a: gpu_runner.to_device(a, "bf16")
    f = workloads.gen_ln_normal(401, 256, 4096, "bf16")
    sp = workloads.gen_rms_uniform(402, 3, 200000, "bf16")
    b = workloads.gen_bwd(403, 512, 2048, "bf16", "ln_bwd")
    lb = workloads.gen_bwd(404, 5, 100000, "bf16", "rms_bwd")    # split backward
    x, g, be = dev(f["x"]).view(256, 4096), dev(f["gamma"]), dev(f["beta"])
    xs, gs = dev(sp["x"]).view(3, 200000), dev(sp["gamma"])
    bx, bg, dy = dev(b["x"]).view(512, 2048), dev(b["gamma"]), dev(b["dy"]).view(512, 2048)
    lx, lg, ldy = dev(lb["x"]).view(5, 100000), dev(lb["gamma"]), dev(lb["dy"]).view(5, 100000)

    def body():
        y, mean, rstd = rn.layer_norm(x, g, be, 1e-5)
        ys, rs = rn.rms_norm(xs, gs, 1e-6)
        _, bm, br = rn.layer_norm(bx, bg, None, 1e-5)
        dx, dg, db = rn.layer_norm_backward(dy, bx, bm, br, bg)
        _, lr = rn.rms_norm(lx, lg, 1e-6)
        ldx, ldg = rn.rms_norm_backward(ldy, lx, lr, lg)
        return [y, mean, rstd, ys, rs, dx, dg, db, lr, ldx, ldg]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):          # warm-up on the capturing stream: workspaces exist
            eager = [t.clone() for t in body()]
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    print("[gpu] capturing", flush=True)
    with torch.cuda.graph(graph, stream=s):
        static = body()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in static:
            t.fill_(float("nan") if t.dtype != torch.int16 else 0)   # make stale outputs visible
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, e) in enumerate(zip(static, eager)):
            assert torch.equal(bits(a), bits(e)), f"replay {rep}: output {k} differs from the eager result"
        # eager work between replays, on the default stream
        junk = rn.layer_norm(x, g, be, 1e-5)[0]
        torch.cuda.synchronize()
        del junk


def test_replay_after_a_larger_eager_call_grew_the_workspace():
    """A graph captured with the split path's workspace keeps using it after a
    larger eager call on the capturing stream replaced it: the old workspace
    is never freed, so the replays still give the eager bits."""
    dev = lambda a: gpu_runner.to_device(a, "bf16")
    small = workloads.gen_ln_normal(411, 2, 100000, "bf16")
    big = workloads.gen_ln_normal(412, 40, 200000, "bf16")
    xs, gs, bs = dev(small["x"]).view(2, 100000), dev(small["gamma"]), dev(small["beta"])
    xb, gb, bb = dev(big["x"]).view(40, 200000), dev(big["gamma"]), dev(big["beta"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        eager = [t.clone() for t in rn.layer_norm(xs, gs, bs, 1e-5)]   # workspace for the small call
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("[gpu] capturing the small split call", flush=True)
    with torch.cuda.graph(graph, stream=s):
        static = rn.layer_norm(xs, gs, bs, 1e-5)
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.cuda.stream(s):
            yb, _, rb = rn.layer_norm(xb, gb, bb, 1e-5)     # larger: a new workspace for s
        torch.cuda.synchronize()
        assert bool(torch.isfinite(rb).all())
        for t in static:
            t.fill_(float("nan"))
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        for k, (a, e) in enumerate(zip(static, eager)):
            assert torch.equal(bits(a), bits(e)), f"replay {rep}: output {k} differs from the eager result"
        del yb, rb
