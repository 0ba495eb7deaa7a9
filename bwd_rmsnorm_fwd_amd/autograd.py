"""torch.autograd integration of the C ABI (the role of P1 §5.5's
autograd.Function and module, "训推加速 Qwen3 实战：从“调包”到手写 Triton
Kernel（含 backward）").

Marshalling only: the forward saves (x, w, rstd) -- the statistic the forward
kernel wrote -- and the backward calls rmsnorm_bwd with it.  Output and
workspace tensors are allocated by torch's caching allocator.  Second-order
gradients are not supported (P1 §5.6's gotcha table): the backward is marked
once-differentiable and raises if differentiated again.
"""
from __future__ import annotations

import torch
from torch.autograd.function import once_differentiable

from . import binding as B


def _workspace(rows: int, H: int, dtype: torch.dtype, device) -> torch.Tensor:
    code = B.F32 if dtype == torch.float32 else B.BF16
    n = B.rmsnorm_bwd_workspace_bytes(rows, H, code)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


class RMSNormFunction(torch.autograd.Function):
    """y = w * x / sqrt(mean(x^2, last dim) + eps)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6):
        H = x.shape[-1]
        x2 = x.contiguous().view(-1, H)
        w = weight.contiguous()
        y = torch.empty_like(x2)
        rstd = torch.empty(x2.shape[0], dtype=torch.float32, device=x.device)
        B.rmsnorm_fwd(x2, w, y, rstd, float(eps))
        ctx.save_for_backward(x2, w, rstd)
        ctx.eps = float(eps)
        ctx.shape = x.shape
        return y.view(x.shape)

    @staticmethod
    @once_differentiable
    def backward(ctx, dy: torch.Tensor):
        x2, w, rstd = ctx.saved_tensors
        dy2 = dy.contiguous().view(x2.shape)
        dx = torch.empty_like(x2)
        dw = torch.empty_like(w)
        ws = _workspace(x2.shape[0], x2.shape[1], x2.dtype, x2.device)
        B.rmsnorm_bwd(dy2, x2, w, rstd, None, dx, dw, ws, ctx.eps)
        return dx.view(ctx.shape), dw, None


class ResidualRMSNormFunction(torch.autograd.Function):
    """(y, h) with h = x + res stored in the I/O dtype and y = RMSNorm(h)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, res: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6):
        H = x.shape[-1]
        x2 = x.contiguous().view(-1, H)
        r2 = res.contiguous().view(-1, H)
        w = weight.contiguous()
        h = torch.empty_like(x2)
        y = torch.empty_like(x2)
        rstd = torch.empty(x2.shape[0], dtype=torch.float32, device=x.device)
        B.rmsnorm_residual_fwd(x2, r2, w, h, y, rstd, float(eps))
        ctx.save_for_backward(h, w, rstd)
        ctx.eps = float(eps)
        ctx.shape = x.shape
        return y.view(x.shape), h.view(x.shape)

    @staticmethod
    @once_differentiable
    def backward(ctx, dy: torch.Tensor, dh_in: torch.Tensor):
        h, w, rstd = ctx.saved_tensors
        dy2 = dy.contiguous().view(h.shape) if dy is not None else torch.zeros_like(h)
        dres = dh_in.contiguous().view(h.shape) if dh_in is not None else None
        dh = torch.empty_like(h)
        dw = torch.empty_like(w)
        ws = _workspace(h.shape[0], h.shape[1], h.dtype, h.device)
        B.rmsnorm_bwd(dy2, h, w, rstd, dres, dh, dw, ws, ctx.eps)
        g = dh.view(ctx.shape)
        return g, g, dw, None


def rms_norm(x, weight, eps: float = 1e-6):
    return RMSNormFunction.apply(x, weight, eps)


def residual_rms_norm(x, res, weight, eps: float = 1e-6):
    """Returns (y, h): the normalised output and the updated residual stream."""
    return ResidualRMSNormFunction.apply(x, res, weight, eps)


class RMSNorm(torch.nn.Module):
    """Module form (weight initialised to ones, as P1 §5.5's module does)."""

    def __init__(self, hidden: int, eps: float = 1e-6, dtype=torch.bfloat16, device="cuda"):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=dtype, device=device))
        self.eps = eps

    def forward(self, x):
        return rms_norm(x, self.weight, self.eps)
