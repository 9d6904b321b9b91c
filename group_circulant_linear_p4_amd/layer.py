"""Drop-in torch layer over the C ABI: the shared parameters w[D', C', T] are the
only state, exactly as in an unrolled ("naive") EQ-Linear layer, so an existing
weight can be used as is ("Implementacao" in "Resumo Tecnico: Flash EQ-Linear":
training-free, plug-and-play replacement).

Forward packs the half spectrum of w and runs eqlinear_fwd; backward runs
eqlinear_bwd_x on the conjugate-transposed packing and eqlinear_bwd_w.  With a bias,
GELU or a residual, the forward is eqlinear_fwd_fused and the backward starts with
eqlinear_fused_epilogue_bwd.  Torch only allocates the buffers; every arithmetic step
runs in the HIP library.
"""
from __future__ import annotations

import math

import torch

from . import (EQL_ACT_GELU, EQL_ACT_NONE, EQL_PACK_BWDX, EQL_PACK_FWD, eqlinear_bwd_w,
               eqlinear_bwd_w_workspace_bytes, eqlinear_bwd_x, eqlinear_fused_epilogue_bwd,
               eqlinear_fused_epilogue_bwd_workspace_bytes, eqlinear_fwd, eqlinear_fwd_fused,
               eqlinear_pack_weight, eqlinear_packed_weight_bytes)


def _packed(w: torch.Tensor, mode: int) -> torch.Tensor:
    Dp, Cp, T = w.shape
    out_ch, in_ch = (Dp, Cp) if mode == EQL_PACK_FWD else (Cp, Dp)
    buf = torch.empty(eqlinear_packed_weight_bytes(out_ch, in_ch, T, w.dtype), dtype=torch.uint8, device=w.device)
    eqlinear_pack_weight(w, buf, Dp, Cp, T, w.dtype, mode)
    return buf


class EQLinearFunction(torch.autograd.Function):
    """y[..., D'*T] = x[..., C'*T] W^T with W[d*T+g, c*T+h] = w[d, c, (g-h) mod T]."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor):
        Dp, Cp, T = w.shape
        if x.shape[-1] != Cp * T:
            raise ValueError("x has %d features, the weight expects C'*T = %d" % (x.shape[-1], Cp * T))
        if x.dtype != w.dtype:
            raise ValueError("x and w must share a dtype (fp16 or fp32)")
        w = w.contiguous()
        x2 = x.reshape(-1, Cp * T).contiguous()
        N = x2.shape[0]
        y = torch.empty((N, Dp * T), dtype=x.dtype, device=x.device)
        eqlinear_fwd(x2, _packed(w, EQL_PACK_FWD), y, N, Cp, Dp, T, x.dtype)
        ctx.save_for_backward(x2, w)
        ctx.lead_shape = x.shape[:-1]
        return y.reshape(*x.shape[:-1], Dp * T)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, w = ctx.saved_tensors
        Dp, Cp, T = w.shape
        N = x2.shape[0]
        dy2 = dy.reshape(-1, Dp * T).to(x2.dtype).contiguous()
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = torch.empty((N, Cp * T), dtype=x2.dtype, device=x2.device)
            eqlinear_bwd_x(dy2, _packed(w, EQL_PACK_BWDX), dx, N, Cp, Dp, T, x2.dtype)
            dx = dx.reshape(*ctx.lead_shape, Cp * T)
        if ctx.needs_input_grad[1]:
            ws_bytes = eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, x2.dtype)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x2.device)
            dw = torch.empty_like(w)
            eqlinear_bwd_w(x2, dy2, dw, ws, ws_bytes, N, Cp, Dp, T, x2.dtype)
        return dx, dw


def eqlinear(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    return EQLinearFunction.apply(x, w)


def _act_code(act):
    if act in (None, "none"):
        return EQL_ACT_NONE
    if act == "gelu":
        return EQL_ACT_GELU
    raise ValueError("activation must be None, 'none' or 'gelu'")


class EQLinearFusedFunction(torch.autograd.Function):
    """y = act(x W^T + b) + r: b[D'] shared by the T group elements of each output
    channel, act none or GELU, r a residual of the output's shape (each optional).

    Forward: one eqlinear_fwd_fused launch, which also keeps the activation's input
    when a gradient will be needed.  Backward: eqlinear_fused_epilogue_bwd (dpre and
    the bias gradient; without an activation dpre is dy itself), then eqlinear_bwd_x
    and eqlinear_bwd_w on dpre; the residual's gradient is dy."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, b, r, act, grad_mode: bool):
        Dp, Cp, T = w.shape
        if x.shape[-1] != Cp * T:
            raise ValueError("x has %d features, the weight expects C'*T = %d" % (x.shape[-1], Cp * T))
        if x.dtype != w.dtype or (b is not None and b.dtype != x.dtype) or (r is not None and r.dtype != x.dtype):
            raise ValueError("x, w, bias and residual must share a dtype (fp16 or fp32)")
        code = _act_code(act)
        w = w.contiguous()
        x2 = x.reshape(-1, Cp * T).contiguous()
        N = x2.shape[0]
        if r is not None and r.numel() != N * Dp * T:
            raise ValueError("residual must have the output's shape")
        r2 = r.reshape(N, Dp * T).contiguous() if r is not None else None
        y = torch.empty((N, Dp * T), dtype=x.dtype, device=x.device)
        # grad_mode is the caller's grad mode (autograd runs this body with grad disabled):
        # pre is kept only when a backward can follow.
        keep = code == EQL_ACT_GELU and grad_mode and any(ctx.needs_input_grad[:3])
        pre = torch.empty_like(y) if keep else None
        eqlinear_fwd_fused(x2, _packed(w, EQL_PACK_FWD), b.contiguous() if b is not None else None, r2, y, pre,
                           N, Cp, Dp, T, x.dtype, code)
        ctx.save_for_backward(x2, w, pre)
        ctx.code, ctx.has_bias, ctx.lead_shape = code, b is not None, x.shape[:-1]
        ctx.res_shape = r.shape if r is not None else None
        return y.reshape(*x.shape[:-1], Dp * T)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, w, pre = ctx.saved_tensors
        Dp, Cp, T = w.shape
        N = x2.shape[0]
        dy2 = dy.reshape(-1, Dp * T).to(x2.dtype).contiguous()
        dr = dy2.reshape(ctx.res_shape) if ctx.res_shape is not None and ctx.needs_input_grad[3] else None
        dx = dw = db = None
        if not any(ctx.needs_input_grad[:3]):
            return dx, dw, db, dr, None, None
        # Without an activation dpre = dy: the call then only sums the bias gradient.
        dpre = torch.empty_like(dy2) if ctx.code == EQL_ACT_GELU else dy2
        if ctx.has_bias and ctx.needs_input_grad[2]:
            db = torch.empty(Dp, dtype=x2.dtype, device=x2.device)
        if ctx.code == EQL_ACT_GELU or db is not None:
            ws_bytes = eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, x2.dtype)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x2.device)
            eqlinear_fused_epilogue_bwd(dy2, pre, dpre, db, ws, ws_bytes, N, Dp, T, x2.dtype, ctx.code)
        if ctx.needs_input_grad[0]:
            dx = torch.empty((N, Cp * T), dtype=x2.dtype, device=x2.device)
            eqlinear_bwd_x(dpre, _packed(w, EQL_PACK_BWDX), dx, N, Cp, Dp, T, x2.dtype)
            dx = dx.reshape(*ctx.lead_shape, Cp * T)
        if ctx.needs_input_grad[1]:
            wsw = eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, x2.dtype)
            wsb = torch.empty(max(wsw, 16), dtype=torch.uint8, device=x2.device)
            dw = torch.empty_like(w)
            eqlinear_bwd_w(x2, dpre, dw, wsb, wsw, N, Cp, Dp, T, x2.dtype)
        return dx, dw, db, dr, None, None


def eqlinear_fused(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
                   residual: torch.Tensor | None = None, act: str = "none") -> torch.Tensor:
    """act(x W^T + bias) + residual with the epilogue fused into the forward kernel
    (eqlinear_fwd_fused), the MLP-block epilogue of the networks the layer is built into
    ("Nivel de Rede").  bias has one value per output channel (shared by its T group
    elements); act is "none" or "gelu"; residual has the output's shape.  Differentiable
    in x, w, bias and residual."""
    return EQLinearFusedFunction.apply(x, w, bias, residual, act, torch.is_grad_enabled())


class EQLinear(torch.nn.Module):
    """Equivariant linear layer over C_T: in_channels*T -> out_channels*T features."""

    def __init__(self, in_channels: int, out_channels: int, group_order: int = 4, bias: bool = False,
                 activation: str | None = None, device=None, dtype=None):
        super().__init__()
        self.in_channels, self.out_channels, self.group_order = in_channels, out_channels, group_order
        _act_code(activation)
        self.activation = activation
        self.weight = torch.nn.Parameter(torch.empty(out_channels, in_channels, group_order, device=device,
                                                     dtype=dtype))
        # One bias per output channel, shared by its group elements (equivariant).
        self.bias = torch.nn.Parameter(torch.zeros(out_channels, device=device, dtype=dtype)) if bias else None
        with torch.no_grad():
            self.weight.normal_(0.0, 1.0 / math.sqrt(in_channels * group_order))

    def forward(self, x: torch.Tensor, residual: torch.Tensor | None = None) -> torch.Tensor:
        """y = act(x W^T + bias) + residual (the parts not configured are skipped)."""
        if self.bias is None and self.activation in (None, "none") and residual is None:
            return EQLinearFunction.apply(x, self.weight)
        return EQLinearFusedFunction.apply(x, self.weight, self.bias, residual, self.activation,
                                           torch.is_grad_enabled())

    def extra_repr(self) -> str:
        return "in_channels=%d, out_channels=%d, group_order=%d, bias=%s, activation=%s" % (
            self.in_channels, self.out_channels, self.group_order, self.bias is not None, self.activation)
