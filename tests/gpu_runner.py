"""Run the library's C ABI on the GPU with numpy-held inputs (test helper)."""
from __future__ import annotations

import numpy as np
import torch

import rmsnorm_forward_amd as rn

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
CODE = {"f32": rn.NORM_F32, "f16": rn.NORM_F16, "bf16": rn.NORM_BF16}
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def to_device(a: np.ndarray, dtype: str, offset: int = 0) -> torch.Tensor:
    """Copy a storage array to the GPU as a flat tensor.  With offset > 0 the
    data starts `offset` elements into a fresh allocation, so its address is
    not 16-byte aligned (the element-wise path)."""
    a = np.ascontiguousarray(a).reshape(-1)
    if dtype == "bf16":
        host = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(a)
    buf = torch.empty(a.size + offset, dtype=TORCH_DT[dtype], device="cuda")
    view = buf[offset:]
    view.copy_(host)
    return view


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def run(op: str, dtype: str, x: np.ndarray, gamma, beta, eps: float, *, stats: bool = True,
        offset: int = 0, keep_device: bool = False):
    """One ln_fwd / rms_fwd call; returns (y, mean, rstd) as host arrays
    (mean is None for RMSNorm or stats=False)."""
    M, N = x.shape
    xt = to_device(x, dtype, offset)
    gt = to_device(gamma, dtype, offset) if gamma is not None else None
    bt = to_device(beta, dtype, offset) if (beta is not None and op == "ln") else None
    ybuf = torch.empty(M * N + offset, dtype=TORCH_DT[dtype], device="cuda")
    yt = ybuf[offset:]
    mean = torch.empty(M, dtype=torch.float32, device="cuda") if (stats and op == "ln") else None
    rstd = torch.empty(M, dtype=torch.float32, device="cuda") if stats else None
    p = lambda t: t.data_ptr() if t is not None else None
    fn = rn.ln_fwd if op == "ln" else rn.rms_fwd
    stream = torch.cuda.current_stream().cuda_stream
    st = fn(p(xt), p(gt), p(bt), p(yt), p(mean), p(rstd), M, N, eps, CODE[dtype], stream)
    assert st == rn.NORM_OK, f"{rn.STATUS.get(st)}: {rn.norm_status_str(st)} [{rn.norm_last_error()}]"
    torch.cuda.synchronize()
    y = to_host(yt, dtype).reshape(M, N)
    m = mean.cpu().numpy() if mean is not None else None
    r = rstd.cpu().numpy() if rstd is not None else None
    if keep_device:
        return y, m, r, (xt, gt, bt, yt, mean, rstd)
    return y, m, r


def run_add(dtype: str, x: np.ndarray, res: np.ndarray, gamma, eps: float, *, stats: bool = True,
            offset: int = 0, inplace: bool = False):
    """One add_rms_fwd call; returns (y, h, rstd) as host arrays.  With
    inplace=True, y is written over x and h over the residual."""
    M, N = x.shape
    xt = to_device(x, dtype, offset)
    rt = to_device(res, dtype, offset)
    gt = to_device(gamma, dtype, offset) if gamma is not None else None
    if inplace:
        yt, ht = xt, rt
    else:
        yt = torch.empty(M * N + offset, dtype=TORCH_DT[dtype], device="cuda")[offset:]
        ht = torch.empty(M * N + offset, dtype=TORCH_DT[dtype], device="cuda")[offset:]
    rstd = torch.empty(M, dtype=torch.float32, device="cuda") if stats else None
    p = lambda t: t.data_ptr() if t is not None else None
    stream = torch.cuda.current_stream().cuda_stream
    st = rn.add_rms_fwd(p(xt), p(rt), p(gt), p(yt), p(ht), p(rstd), M, N, eps, CODE[dtype], stream)
    assert st == rn.NORM_OK, f"{rn.STATUS.get(st)}: {rn.norm_status_str(st)} [{rn.norm_last_error()}]"
    torch.cuda.synchronize()
    y = to_host(yt, dtype).reshape(M, N)
    h = to_host(ht, dtype).reshape(M, N)
    r = rstd.cpu().numpy() if rstd is not None else None
    return y, h, r


def run_fp8(dtype: str, x: np.ndarray, res, gamma, eps: float, scale: float, *, stats: bool = True,
            offset: int = 0, inplace: bool = False):
    """One rms_fp8_fwd (res None) or add_rms_fp8_fwd call; returns (codes
    uint8, h or None, rstd) as host arrays."""
    M, N = x.shape
    xt = to_device(x, dtype, offset)
    rt = to_device(res, dtype, offset) if res is not None else None
    gt = to_device(gamma, dtype, offset) if gamma is not None else None
    qt = torch.zeros(M * N + 16, dtype=torch.uint8, device="cuda")[offset:offset + M * N]
    ht = None
    if res is not None:
        ht = rt if inplace else torch.empty(M * N + offset, dtype=TORCH_DT[dtype], device="cuda")[offset:]
    rstd = torch.empty(M, dtype=torch.float32, device="cuda") if stats else None
    p = lambda t: t.data_ptr() if t is not None else None
    stream = torch.cuda.current_stream().cuda_stream
    if res is None:
        st = rn.rms_fp8_fwd(p(xt), p(gt), p(qt), p(rstd), M, N, eps, scale, CODE[dtype], stream)
    else:
        st = rn.add_rms_fp8_fwd(p(xt), p(rt), p(gt), p(qt), p(ht), p(rstd), M, N, eps, scale, CODE[dtype],
                                stream)
    assert st == rn.NORM_OK, f"{rn.STATUS.get(st)}: {rn.norm_status_str(st)} [{rn.norm_last_error()}]"
    torch.cuda.synchronize()
    q = qt.cpu().numpy().reshape(M, N)
    h = to_host(ht, dtype).reshape(M, N) if ht is not None else None
    r = rstd.cpu().numpy() if rstd is not None else None
    return q, h, r


def run_bwd(op: str, dtype: str, dy: np.ndarray, x: np.ndarray, gamma, mean, rstd, *, offset: int = 0,
            inplace: str | None = None, want_g: bool = True, want_b: bool = True):
    """One ln_bwd / rms_bwd call on host arrays (mean / rstd: fp32 [M]);
    returns (dx, dgamma, dbeta) as host arrays (None where not asked for).
    inplace = "dy" or "x" writes dx over that input."""
    M, N = x.shape
    dyt = to_device(dy, dtype, offset)
    xt = to_device(x, dtype, offset)
    gt = to_device(gamma, dtype, offset) if gamma is not None else None
    mt = torch.from_numpy(np.ascontiguousarray(mean, np.float32)).cuda() if op == "ln" else None
    rt = torch.from_numpy(np.ascontiguousarray(rstd, np.float32)).cuda()
    if inplace == "dy":
        dxt = dyt
    elif inplace == "x":
        dxt = xt
    else:
        dxt = torch.empty(M * N + offset, dtype=TORCH_DT[dtype], device="cuda")[offset:]
    dgt = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda") if want_g else None
    dbt = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda") if (want_b and op == "ln") else None
    p = lambda t: t.data_ptr() if t is not None else None
    stream = torch.cuda.current_stream().cuda_stream
    if op == "ln":
        st = rn.ln_bwd(p(dyt), p(xt), p(gt), p(mt), p(rt), p(dxt), p(dgt), p(dbt), M, N, CODE[dtype], stream)
    else:
        st = rn.rms_bwd(p(dyt), p(xt), p(gt), p(rt), p(dxt), p(dgt), M, N, CODE[dtype], stream)
    assert st == rn.NORM_OK, f"{rn.STATUS.get(st)}: {rn.norm_status_str(st)} [{rn.norm_last_error()}]"
    torch.cuda.synchronize()
    dx = to_host(dxt, dtype).reshape(M, N)
    dg = dgt.cpu().numpy() if dgt is not None else None
    db = dbt.cpu().numpy() if dbt is not None else None
    return dx, dg, db


def _embed(a: np.ndarray, dtype: str, ld: int, offset: int, fill_bits: int):
    """Device buffer holding the [M, N] storage array `a` with rows `ld`
    elements apart, starting `offset` elements in; every other element holds
    the bit pattern fill_bits.  Returns (buffer, view of the first element)."""
    M, N = a.shape
    tdt = TORCH_DT[dtype] if dtype != "u8" else torch.uint8
    n = offset + (M - 1) * ld + N if M else offset
    host = np.empty(n + 8, NP_STORAGE.get(dtype, np.uint8))
    host.view(np.uint8 if dtype == "u8" else (np.uint32 if dtype == "f32" else np.uint16))[:] = fill_bits
    for r in range(M):
        host[offset + r * ld: offset + r * ld + N] = a[r]
    if dtype == "bf16":
        t = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(host)
    buf = t.to("cuda")
    return buf, buf[offset:]


def _extract(buf, dtype: str, M: int, N: int, ld: int, offset: int):
    """Rows out of a strided buffer, and the buffer's bytes outside the rows."""
    h = buf.cpu()
    if dtype == "bf16":
        h = h.view(torch.int16).numpy().view(np.uint16)
    else:
        h = h.numpy()
    rows = np.stack([h[offset + r * ld: offset + r * ld + N] for r in range(M)]) if M else h[:0]
    mask = np.ones(h.size, bool)
    for r in range(M):
        mask[offset + r * ld: offset + r * ld + N] = False
    return rows, h[mask]


FILL = {"f32": 0x7FA5A5A5, "bf16": 0x7FA5, "f16": 0x7E5A, "u8": 0xA5}


def run_strided(op: str, dtype: str, x, gamma, beta, eps: float, *, res=None, scale: float = 1.0,
                ldx: int, ldy: int, ldr: int = 0, ldh: int = 0, offset: int = 0, inplace: bool = False,
                x_offset: int | None = None):
    """One norm_fwd call with strided rows.  Returns (y, h, mean, rstd) and
    asserts that no byte between or around the rows of the outputs changed.
    x_offset (default: offset) places x alone that many elements into its
    allocation."""
    M, N = x.shape
    q8 = op.endswith("fp8")
    ydt = "u8" if q8 else dtype
    xb, xt = _embed(x, dtype, ldx, offset if x_offset is None else x_offset, FILL[dtype])
    gt = to_device(gamma, dtype) if gamma is not None else None
    bt = to_device(beta, dtype) if beta is not None else None
    rb = rt = hb = ht = None
    if res is not None:
        rb, rt = _embed(res, dtype, ldr or N, offset, FILL[dtype])
        if inplace:
            hb, ht, ldh = rb, rt, (ldr or N)
        else:
            hb, ht = _embed(np.zeros((M, N), NP_STORAGE[dtype]), dtype, ldh or N, offset, FILL[dtype])
    if inplace and not q8:
        yb, yt = xb, xt
    else:
        yb, yt = _embed(np.zeros((M, N), np.uint8 if q8 else NP_STORAGE[dtype]), ydt, ldy, offset, FILL[ydt])
    mean = torch.empty(M, dtype=torch.float32, device="cuda") if op == "ln" else None
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    p = lambda t: t.data_ptr() if t is not None else None
    st = rn.norm_fwd(op, CODE[dtype], M, N, p(xt), p(yt), ld_x=ldx, residual=p(rt), ld_residual=ldr,
                     gamma=p(gt), beta=p(bt), ld_y=ldy, residual_out=p(ht), ld_residual_out=ldh,
                     mean=p(mean), rstd=p(rstd), eps=eps, scale=scale,
                     stream=torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_OK, f"{rn.STATUS.get(st)}: {rn.norm_status_str(st)} [{rn.norm_last_error()}]"
    torch.cuda.synchronize()
    def bits(a, dt):
        return a.view({"f32": np.uint32, "f16": np.uint16}.get(dt, a.dtype))

    y, ygap = _extract(yb, ydt, M, N, ldy, offset)
    assert np.all(bits(ygap, ydt) == FILL[ydt]), "a write landed outside the rows of y"
    h = None
    if ht is not None:
        h, hgap = _extract(hb, dtype, M, N, ldh or N, offset)
        assert np.all(bits(hgap, dtype) == FILL[dtype]), "a write landed outside the rows of the residual sum"
    return (y, h, mean.cpu().numpy() if mean is not None else None, rstd.cpu().numpy())


def run_bwd_strided(op: str, dtype: str, dy, x, gamma, mean, rstd, *, lddy: int, ldx: int, lddx: int,
                    offset: int = 0, inplace: str | None = None):
    """One norm_bwd call with strided rows.  Returns (dx, dgamma, dbeta) and
    asserts that no byte between or around the rows of dx changed (and,
    unless dx is written over it, that dy and x are unchanged)."""
    M, N = x.shape
    dyb, dyt = _embed(dy, dtype, lddy, offset, FILL[dtype])
    xb, xt = _embed(x, dtype, ldx, offset, FILL[dtype])
    gt = to_device(gamma, dtype) if gamma is not None else None
    mt = torch.from_numpy(np.ascontiguousarray(mean, np.float32)).cuda() if op == "ln" else None
    rt = torch.from_numpy(np.ascontiguousarray(rstd, np.float32)).cuda()
    if inplace == "dy":
        dxb, dxt, lddx = dyb, dyt, lddy
    elif inplace == "x":
        dxb, dxt, lddx = xb, xt, ldx
    else:
        dxb, dxt = _embed(np.zeros((M, N), NP_STORAGE[dtype]), dtype, lddx, offset, FILL[dtype])
    dgt = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    dbt = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda") if op == "ln" else None
    p = lambda t: t.data_ptr() if t is not None else None
    st = rn.norm_bwd(op, CODE[dtype], M, N, p(dyt), p(xt), p(dxt), ld_dy=lddy, ld_x=ldx, ld_dx=lddx,
                     gamma=p(gt), mean=p(mt), rstd=p(rt), dgamma=p(dgt), dbeta=p(dbt),
                     stream=torch.cuda.current_stream().cuda_stream)
    assert st == rn.NORM_OK, f"{rn.STATUS.get(st)}: {rn.norm_status_str(st)} [{rn.norm_last_error()}]"
    torch.cuda.synchronize()
    bits = lambda a: a.view({"f32": np.uint32, "f16": np.uint16}.get(dtype, a.dtype))
    dx, gap = _extract(dxb, dtype, M, N, lddx, offset)
    assert np.all(bits(gap) == FILL[dtype]), "a write landed outside the rows of dx"
    for name, (b, a, ld) in {"dy": (dyb, dy, lddy), "x": (xb, x, ldx)}.items():
        if inplace == name:
            continue
        rows, _ = _extract(b, dtype, M, N, ld, offset)
        assert np.array_equal(bits(rows), bits(np.ascontiguousarray(a))), f"{name} changed"
    return dx, dgt.cpu().numpy(), dbt.cpu().numpy() if dbt is not None else None
