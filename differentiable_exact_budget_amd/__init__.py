"""Fast LapSum on MI355X: exact-budget differentiable soft top-k.

    p = soft_topk(r, k, t)      # sum(p) == k, p_i = F((r_i - b)/t), F the Laplace CDF

The forward solve and the analytic VJP run in liblapsum.so (hand-written HIP
for gfx950); this package only marshals torch tensors into the C ABI of
include/lapsum.h.  It raises if the library is not built -- there is no CPU
or PyTorch fallback.
"""
import ctypes

import torch

from ._binding import (PATH_AUTO, PATH_BRACKET, PATH_FORCE_FALLBACK, PATH_FULL, LapsumError, Options, Stats,
                       default_options, lib)

__all__ = ["forward", "vjp", "vjp_kt", "soft_topk", "topk_threshold", "hard_topk", "dftopk",
           "forward_rows", "vjp_rows", "soft_topk_rows", "SoftTopK", "default_options", "Options", "Stats", "LapsumError",
           "PATH_AUTO", "PATH_FULL", "PATH_BRACKET", "PATH_FORCE_FALLBACK", "release_workspaces"]


def _check_scores(x: torch.Tensor, name: str) -> None:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {x.device})")
    if x.dtype != torch.float32:
        raise ValueError(f"{name} must be float32 (got {x.dtype})")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def forward(r: torch.Tensor, k: float, t: float, *, options: Options = None, stats: bool = False,
            p_out: torch.Tensor = None, b_out: torch.Tensor = None):
    """Solve the exact-budget threshold and write p.

    Returns (p, b) -- b is a 1-element float64 tensor on the same device --
    or (p, b, stats_dict) when stats=True (which waits for the device)."""
    _check_scores(r, "r")
    n = r.numel()
    with torch.cuda.device(r.device):
        p = p_out if p_out is not None else torch.empty_like(r)
        b = b_out if b_out is not None else torch.empty(1, dtype=torch.float64, device=r.device)
        _check_scores(p, "p_out")
        if b.dtype != torch.float64 or b.device != r.device or b.numel() < 1:
            raise ValueError("b_out must be a float64 tensor with one element on r's device")
        st = Stats() if stats else None
        rc = lib().lapsum_forward_ex(r.data_ptr(), n, float(k), float(t), p.data_ptr(), b.data_ptr(),
                                     ctypes.byref(options) if options is not None else None,
                                     ctypes.byref(st) if st is not None else None, _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_forward")
    if stats:
        return p, b, st.as_dict()
    return p, b


def vjp(r: torch.Tensor, g: torch.Tensor, t: float, b: torch.Tensor, *, grad_out: torch.Tensor = None,
        options: Options = None, stats: bool = False):
    """grad_i = (f_i/t)(g_i - sum g f / sum f), f_i = e^{-|r_i - b|/t}/2.
    Returns grad, or (grad, stats_dict) when stats=True (which waits)."""
    _check_scores(r, "r")
    _check_scores(g, "g")
    if g.numel() != r.numel():
        raise ValueError("g must have as many elements as r")
    if b.dtype != torch.float64 or b.device != r.device:
        raise ValueError("b must be the float64 device tensor returned by forward")
    with torch.cuda.device(r.device):
        out = grad_out if grad_out is not None else torch.empty_like(r)
        _check_scores(out, "grad_out")
        st = Stats() if stats else None
        rc = lib().lapsum_vjp_ex(r.data_ptr(), None, g.data_ptr(), r.numel(), float(t), b.data_ptr(), out.data_ptr(),
                                 ctypes.byref(options) if options is not None else None,
                                 ctypes.byref(st) if st is not None else None, _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_vjp")
    if stats:
        return out, st.as_dict()
    return out


def vjp_kt(r: torch.Tensor, g: torch.Tensor, t: float, b: torch.Tensor, *, want_grad: bool = True,
           grad_out: torch.Tensor = None, options: Options = None, stats: bool = False):
    """The VJP together with dL/dk and dL/dt (L = sum g p).

    Returns (grad, dk, dt): grad as in vjp (None when want_grad is False:
    then a single pass over r and g forms the scalars), dk and dt 1-element
    float64 device tensors; plus a stats dict when stats=True (which waits)."""
    _check_scores(r, "r")
    _check_scores(g, "g")
    if g.numel() != r.numel():
        raise ValueError("g must have as many elements as r")
    if b.dtype != torch.float64 or b.device != r.device:
        raise ValueError("b must be the float64 device tensor returned by forward")
    with torch.cuda.device(r.device):
        out = None
        if want_grad:
            out = grad_out if grad_out is not None else torch.empty_like(r)
            _check_scores(out, "grad_out")
        dk = torch.empty(1, dtype=torch.float64, device=r.device)
        dt = torch.empty(1, dtype=torch.float64, device=r.device)
        st = Stats() if stats else None
        rc = lib().lapsum_vjp_kt(r.data_ptr(), g.data_ptr(), r.numel(), float(t), b.data_ptr(),
                                 out.data_ptr() if out is not None else None, dk.data_ptr(), dt.data_ptr(),
                                 ctypes.byref(options) if options is not None else None,
                                 ctypes.byref(st) if st is not None else None, _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_vjp_kt")
    if stats:
        return out, dk, dt, st.as_dict()
    return out, dk, dt


class SoftTopK(torch.autograd.Function):
    """Autograd wrapper: forward solves for b and writes p; backward is the
    analytic VJP with respect to the scores, and with respect to k and t
    when those are tensors that require a gradient."""

    @staticmethod
    def forward(ctx, r, k, t, options=None):
        rc = r.contiguous()
        p, b = forward(rc, float(k), float(t), options=options)
        ctx.save_for_backward(rc, b)
        ctx.t = float(t)
        ctx.k_meta = (k.shape, k.dtype, k.device) if isinstance(k, torch.Tensor) else None
        ctx.t_meta = (t.shape, t.dtype, t.device) if isinstance(t, torch.Tensor) else None
        return p

    @staticmethod
    def backward(ctx, g):
        r, b = ctx.saved_tensors
        g32 = g.contiguous().to(torch.float32)
        need_r, need_k, need_t = ctx.needs_input_grad[0], ctx.needs_input_grad[1], ctx.needs_input_grad[2]
        if not (need_k or need_t):
            return vjp(r, g32, ctx.t, b), None, None, None
        grad, dk, dt = vjp_kt(r, g32, ctx.t, b, want_grad=need_r)

        def like(x, meta):
            shape, dtype, device = meta
            return x.to(device=device, dtype=dtype).reshape(shape)

        return (grad, like(dk, ctx.k_meta) if need_k else None, like(dt, ctx.t_meta) if need_t else None, None)


def soft_topk(r: torch.Tensor, k, t, options: Options = None) -> torch.Tensor:
    """Differentiable exact-budget soft top-k over a flat fp32 tensor.  k and t
    are numbers, or one-element tensors when their gradients are wanted."""
    shape = r.shape
    p = SoftTopK.apply(r.reshape(-1), k, t, options)
    return p.reshape(shape)


def _opts(options):
    return ctypes.byref(options) if options is not None else None


def topk_threshold(r: torch.Tensor, k: int, *, options: Options = None, stats: bool = False):
    """(k-th largest, (k+1)-th largest) of r as a 2-element float64 device
    tensor (the second is -inf when k = n)."""
    _check_scores(r, "r")
    with torch.cuda.device(r.device):
        tau = torch.empty(2, dtype=torch.float64, device=r.device)
        st = Stats() if stats else None
        rc = lib().lapsum_topk_threshold(r.data_ptr(), r.numel(), int(k), tau.data_ptr(), _opts(options),
                                         ctypes.byref(st) if st is not None else None, _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_topk_threshold")
    return (tau, st.as_dict()) if stats else tau


def hard_topk(r: torch.Tensor, k: int, *, options: Options = None, stats: bool = False):
    """mask (fp32, 1 where r >= the k-th largest) and the two order statistics."""
    _check_scores(r, "r")
    with torch.cuda.device(r.device):
        mask = torch.empty_like(r)
        tau = torch.empty(2, dtype=torch.float64, device=r.device)
        st = Stats() if stats else None
        rc = lib().lapsum_hard_topk(r.data_ptr(), r.numel(), int(k), mask.data_ptr(), tau.data_ptr(), _opts(options),
                                    ctypes.byref(st) if st is not None else None, _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_hard_topk")
    return (mask, tau, st.as_dict()) if stats else (mask, tau)


def dftopk(r: torch.Tensor, k: int, t: float, *, options: Options = None, stats: bool = False):
    """DFTopK: b = midpoint of the k-th and (k+1)-th largest, p = F((r - b)/t).
    Returns (p, b) with b a 1-element float64 device tensor."""
    _check_scores(r, "r")
    with torch.cuda.device(r.device):
        p = torch.empty_like(r)
        b = torch.empty(1, dtype=torch.float64, device=r.device)
        st = Stats() if stats else None
        rc = lib().lapsum_dftopk(r.data_ptr(), r.numel(), int(k), float(t), p.data_ptr(), b.data_ptr(),
                                 _opts(options), ctypes.byref(st) if st is not None else None, _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_dftopk")
    return (p, b, st.as_dict()) if stats else (p, b)


def forward_rows(r: torch.Tensor, k, t: float):
    """Row-wise solve of a 2-D fp32 tensor [rows, n]: k is a number or a
    float64 tensor of rows budgets on r's device.  Returns (p, b), b float64[rows]."""
    _check_scores(r, "r")
    if r.dim() != 2:
        raise ValueError("r must be 2-D [rows, n]")
    rows, n = r.shape
    with torch.cuda.device(r.device):
        p = torch.empty_like(r)
        b = torch.empty(rows, dtype=torch.float64, device=r.device)
        if isinstance(k, torch.Tensor):
            kr = k.to(device=r.device, dtype=torch.float64).contiguous()
            if kr.numel() != rows:
                raise ValueError("k must have one budget per row")
            rc = lib().lapsum_forward_batched(r.data_ptr(), rows, n, 0.0, kr.data_ptr(), float(t), p.data_ptr(),
                                              b.data_ptr(), _stream_ptr(r.device))
        else:
            rc = lib().lapsum_forward_batched(r.data_ptr(), rows, n, float(k), None, float(t), p.data_ptr(),
                                              b.data_ptr(), _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_forward_batched")
    return p, b


def vjp_rows(r: torch.Tensor, g: torch.Tensor, t: float, b: torch.Tensor):
    """Row-wise VJP: grad[i] = (f/t)(g[i] - sum g f / sum f) within row i."""
    _check_scores(r, "r")
    _check_scores(g, "g")
    if r.dim() != 2 or g.shape != r.shape:
        raise ValueError("r and g must be 2-D tensors of one shape")
    if b.dtype != torch.float64 or b.numel() != r.shape[0]:
        raise ValueError("b must be the float64[rows] tensor returned by forward_rows")
    with torch.cuda.device(r.device):
        out = torch.empty_like(r)
        rc = lib().lapsum_vjp_batched(r.data_ptr(), g.data_ptr(), r.shape[0], r.shape[1], float(t), b.data_ptr(),
                                      out.data_ptr(), _stream_ptr(r.device))
    if rc != 0:
        raise LapsumError(rc, "lapsum_vjp_batched")
    return out


class SoftTopKRows(torch.autograd.Function):
    """Row-wise exact-budget soft top-k with the analytic VJP per row."""

    @staticmethod
    def forward(ctx, r, k, t):
        rc = r.contiguous()
        p, b = forward_rows(rc, k, t)
        ctx.save_for_backward(rc, b)
        ctx.t = float(t)
        return p

    @staticmethod
    def backward(ctx, g):
        r, b = ctx.saved_tensors
        return vjp_rows(r, g.contiguous().to(torch.float32), ctx.t, b), None, None


def soft_topk_rows(r: torch.Tensor, k, t: float) -> torch.Tensor:
    """Differentiable exact-budget soft top-k along the last dimension."""
    shape = r.shape
    p = SoftTopKRows.apply(r.reshape(-1, shape[-1]), k, t)
    return p.reshape(shape)


def release_workspaces() -> None:
    lib().lapsum_release_workspaces()
