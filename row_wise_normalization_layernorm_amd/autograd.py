"""Differentiable LayerNorm and RMSNorm over torch tensors.

Both directions run in libmi_norm.so: the forward keeps each row's mean and
rstd (float32), and the backward computes dx and the parameter gradients
from them (mi_norm_bwd).  Rows are the last dimension of a float32, float16
or bfloat16 device tensor; the parameters are float32, as in mi_norm.h.
"""
from __future__ import annotations

import torch

from . import _binding as B


def _last_contiguous(t):
    return t if t.dim() == 0 or t.shape[-1] <= 1 or t.stride(-1) == 1 else t.contiguous()


class _LayerNorm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, eps):
        x = _last_contiguous(x)
        y, mean, rstd = B.layernorm(x, weight, bias, eps, stats=True)
        ctx.save_for_backward(x, weight, mean, rstd)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, weight, mean, rstd = ctx.saved_tensors
        want_p = ctx.needs_input_grad[1] or ctx.needs_input_grad[2]
        dx, dw, db = B.layernorm_bwd(_last_contiguous(dy), x, weight, mean, rstd, param_grads=want_p)
        return (dx, dw if ctx.needs_input_grad[1] else None, db if ctx.needs_input_grad[2] else None, None)


class _RMSNorm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, eps):
        x = _last_contiguous(x)
        y, rstd = B.rmsnorm(x, weight, eps, stats=True)
        ctx.save_for_backward(x, weight, rstd)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, weight, rstd = ctx.saved_tensors
        dx, dw = B.rmsnorm_bwd(_last_contiguous(dy), x, weight, rstd, param_grads=ctx.needs_input_grad[1])
        return dx, dw if ctx.needs_input_grad[1] else None, None


def layer_norm(x, weight, bias, eps: float = 1e-5):
    """y = (x - mean) * rstd * weight + bias over the last dimension, with autograd."""
    return _LayerNorm.apply(x, weight, bias, eps)


def rms_norm(x, weight, eps: float = 1e-5):
    """y = x * rstd * weight over the last dimension, with autograd."""
    return _RMSNorm.apply(x, weight, eps)


class LayerNorm(torch.nn.Module):
    """LayerNorm over the last dimension (d) with float32 weight and bias."""

    def __init__(self, d: int, eps: float = 1e-5, device=None):
        super().__init__()
        self.eps = eps
        self.weight = torch.nn.Parameter(torch.ones(d, device=device, dtype=torch.float32))
        self.bias = torch.nn.Parameter(torch.zeros(d, device=device, dtype=torch.float32))

    def forward(self, x):
        return layer_norm(x, self.weight, self.bias, self.eps)


class RMSNorm(torch.nn.Module):
    """RMSNorm over the last dimension (d) with a float32 weight."""

    def __init__(self, d: int, eps: float = 1e-5, device=None):
        super().__init__()
        self.eps = eps
        self.weight = torch.nn.Parameter(torch.ones(d, device=device, dtype=torch.float32))

    def forward(self, x):
        return rms_norm(x, self.weight, self.eps)
