"""torch.autograd wrapper over the C-ABI forward and backward.

The pages expose the training RMSNorm to autograd through a Function class
and a functional entry point, both taking ``deterministic`` (p1 #8208 PR
description: cake_rmsnorm, CakeRMSNormFunction).  Their measured op
"2xfwd+bwd" is the checkpointed step -- forward, forward recompute,
backward (p2 "Key") -- which ``recompute=True`` gives here: the forward keeps
only its inputs and the backward runs the forward again before the backward
kernel.

Gradient dtypes follow autograd's rule (a gradient has its tensor's dtype):
the weight gradient is the library's FP32 dw, cast to w's dtype when w is
BF16.  Call ``rmsnorm_bwd`` directly to keep the FP32 dw.
"""
from __future__ import annotations

import torch

from . import geometry, rmsnorm_bwd, rmsnorm_fwd, rmsnorm_gated_bwd, rmsnorm_gated_fwd


def _like_layout(t, ref):
    """t with ref's shape and strides (the ABI shares strides between all
    activation tensors); copies only when the layouts differ."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16 and t.shape == ref.shape and geometry(t) == geometry(ref):
        return t
    out = torch.empty_strided(ref.shape, ref.stride(), dtype=torch.bfloat16, device=ref.device)
    out.copy_(t)
    return out


def _rows(t):
    """t as the library sees it: [T,H] or [T,heads,H] pass through; more
    leading dimensions are folded into rows (a view when the strides allow
    it, else a contiguous copy)."""
    if t is None or t.dim() <= 3:
        return t
    try:
        return t.view(-1, t.shape[-1])
    except RuntimeError:
        return t.reshape(-1, t.shape[-1])


class RMSNormFunction(torch.autograd.Function):
    """y = RMSNorm(x [+ residual]) * w.  Returns y, or (y, h) with a residual,
    where h = x + residual is the BF16 residual stream.  x may have any number
    of leading dimensions; the last one is H."""

    @staticmethod
    def forward(ctx, x, w, residual, eps, deterministic, recompute):
        ctx.shape = x.shape
        x, residual = _rows(x), _rows(residual)
        ctx.set_materialize_grads(False)
        y, rstd, h = rmsnorm_fwd(x, w, eps, residual=residual, deterministic=deterministic)
        ctx.eps, ctx.deterministic, ctx.recompute = eps, deterministic, recompute
        ctx.has_residual = residual is not None
        if recompute:
            ctx.save_for_backward(x, w, residual)
        else:
            ctx.save_for_backward(h if residual is not None else x, w, rstd)
        if residual is not None:
            return y.view(ctx.shape), h.view(ctx.shape)
        return y.view(ctx.shape)

    @staticmethod
    def backward(ctx, dy, dh=None):
        dy, dh = _rows(dy), _rows(dh)
        if ctx.recompute:
            x, w, residual = ctx.saved_tensors
            _, rstd, h = rmsnorm_fwd(x, w, ctx.eps, residual=residual, deterministic=ctx.deterministic)
            u = h if residual is not None else x
        else:
            u, w, rstd = ctx.saved_tensors
        if dy is None:  # only h was used downstream
            dy = torch.zeros_like(u)
        dy = _like_layout(dy, u)
        dres = _like_layout(dh, u) if ctx.has_residual and dh is not None else None
        dx, dw = rmsnorm_bwd(dy, u, rstd, w, residual=dres, deterministic=ctx.deterministic)
        grad_w = dw if w.dtype == torch.float32 else dw.to(w.dtype)
        dx = dx.view(ctx.shape)
        grad_res = dx if ctx.has_residual else None
        return dx, grad_w, grad_res, None, None, None


def rmsnorm(x, w, eps: float = 1e-6, residual=None, deterministic: bool = True,
            recompute: bool = False):
    """Functional form of :class:`RMSNormFunction`."""
    return RMSNormFunction.apply(x, w, residual, eps, deterministic, recompute)


class RMSNorm(torch.nn.Module):
    """Module holding the weight (BF16 or FP32, initialised to ones)."""

    def __init__(self, hidden: int, eps: float = 1e-6, dtype=torch.bfloat16, device=None,
                 deterministic: bool = True, recompute: bool = False):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=dtype, device=device))
        self.eps, self.deterministic, self.recompute = eps, deterministic, recompute

    def forward(self, x, residual=None):
        return rmsnorm(x, self.weight, self.eps, residual, self.deterministic, self.recompute)


class GatedRMSNormFunction(torch.autograd.Function):
    """y = RMSNorm(x) * w * silu(g): the SiLU-gated variant (gradients for
    x, w and g)."""

    @staticmethod
    def forward(ctx, x, g, w, eps, deterministic, recompute):
        ctx.shape = x.shape
        x, g = _rows(x), _rows(g)
        ctx.set_materialize_grads(False)
        y, rstd = rmsnorm_gated_fwd(x, g, w, eps, deterministic=deterministic)
        ctx.eps, ctx.deterministic, ctx.recompute = eps, deterministic, recompute
        ctx.save_for_backward(x, g, w, None if recompute else rstd)
        return y.view(ctx.shape)

    @staticmethod
    def backward(ctx, dy):
        x, g, w, rstd = ctx.saved_tensors
        if dy is None:
            return None, None, None, None, None, None
        if ctx.recompute:
            _, rstd = rmsnorm_gated_fwd(x, g, w, ctx.eps, deterministic=ctx.deterministic)
        dy = _like_layout(_rows(dy), x)
        dx, dg, dw = rmsnorm_gated_bwd(dy, x, g, rstd, w, deterministic=ctx.deterministic)
        grad_w = dw if w.dtype == torch.float32 else dw.to(w.dtype)
        return dx.view(ctx.shape), dg.view(ctx.shape), grad_w, None, None, None


def rmsnorm_gated(x, g, w, eps: float = 1e-6, deterministic: bool = True, recompute: bool = False):
    """Functional form of :class:`GatedRMSNormFunction`."""
    return GatedRMSNormFunction.apply(x, g, w, eps, deterministic, recompute)
