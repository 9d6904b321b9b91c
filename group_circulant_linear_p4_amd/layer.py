"""Drop-in torch layer over the C ABI: the shared parameters w[D', C', T] are the
only state, exactly as in an unrolled ("naive") EQ-Linear layer, so an existing
weight can be used as is ("Implementacao" in "Resumo Tecnico: Flash EQ-Linear":
training-free, plug-and-play replacement).

Forward packs the half spectrum of w and runs eqlinear_fwd; backward runs
eqlinear_bwd_x on the conjugate-transposed packing and eqlinear_bwd_w.  When the weight
needs a gradient, the three passes are the training entry points instead
(eqlinear_fwd_train, eqlinear_bwd_x_train, eqlinear_bwd_w_train): the forward keeps the
weight-gradient workspace, holding x's half spectrum, alive until the backward.  EQLinearP4M is the
layer over p4m's point group (rotations and reflections), run through the same kernels on
the C_4 view described in include/eqlinear.h.  With a bias,
GELU or a residual, the forward is eqlinear_fwd_fused (eqlinear_fwd_fused_train when the
weight needs a gradient) and the backward starts with eqlinear_fused_epilogue_bwd.  Torch only allocates the buffers; every arithmetic step
runs in the HIP library.
"""
from __future__ import annotations

import math

import torch

from . import (EQL_ACT_GELU, EQL_ACT_NONE, EQL_PACK_BWDX, EQL_PACK_FWD, eqlinear_bwd_w,
               eqlinear_bwd_w_train, eqlinear_bwd_w_workspace_bytes, eqlinear_bwd_x,
               eqlinear_bwd_x_train, eqlinear_fused_epilogue_bwd, eqlinear_fwd_fused_train, eqlinear_fwd_train,
               eqlinear_fused_epilogue_bwd_workspace_bytes, eqlinear_fwd, eqlinear_fwd_fused,
               eqlinear_p4m_expand_weight, eqlinear_p4m_fold_weight_grad, eqlinear_pack_weight,
               eqlinear_packed_weight_bytes)


def _packed(w: torch.Tensor, mode: int) -> torch.Tensor:
    Dp, Cp, T = w.shape
    out_ch, in_ch = (Dp, Cp) if mode == EQL_PACK_FWD else (Cp, Dp)
    buf = torch.empty(eqlinear_packed_weight_bytes(out_ch, in_ch, T, w.dtype), dtype=torch.uint8, device=w.device)
    eqlinear_pack_weight(w, buf, Dp, Cp, T, w.dtype, mode)
    return buf


class EQLinearFunction(torch.autograd.Function):
    """y[..., D'*T] = x[..., C'*T] W^T with W[d*T+g, c*T+h] = w[d, c, (g-h) mod T]."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, keep_spectra: bool = True):
        Dp, Cp, T = w.shape
        if x.shape[-1] != Cp * T:
            raise ValueError("x has %d features, the weight expects C'*T = %d" % (x.shape[-1], Cp * T))
        if x.dtype != w.dtype:
            raise ValueError("x and w must share a dtype (fp16 or fp32)")
        w = w.contiguous()
        x2 = x.reshape(-1, Cp * T).contiguous()
        N = x2.shape[0]
        y = torch.empty((N, Dp * T), dtype=x.dtype, device=x.device)
        ws_bytes = eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, x.dtype)
        if keep_spectra and ctx.needs_input_grad[1]:
            # The weight gradient will follow: keep x's spectrum in its workspace.
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
            eqlinear_fwd_train(x2, _packed(w, EQL_PACK_FWD), y, ws, ws_bytes, N, Cp, Dp, T, x.dtype)
        else:
            ws = None
            eqlinear_fwd(x2, _packed(w, EQL_PACK_FWD), y, N, Cp, Dp, T, x.dtype)
        ctx.save_for_backward(x2, w, ws)
        ctx.ws_bytes = ws_bytes
        ctx.lead_shape = x.shape[:-1]
        return y.reshape(*x.shape[:-1], Dp * T)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, w, ws = ctx.saved_tensors
        Dp, Cp, T = w.shape
        N = x2.shape[0]
        dy2 = dy.reshape(-1, Dp * T).to(x2.dtype).contiguous()
        dx = dw = None
        need_dx, need_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        train = ws is not None
        if need_dx:
            dx = torch.empty((N, Cp * T), dtype=x2.dtype, device=x2.device)
            if train and need_dw:  # also leaves dy's spectrum where the weight gradient reads it
                eqlinear_bwd_x_train(dy2, _packed(w, EQL_PACK_BWDX), dx, ws, ctx.ws_bytes, N, Cp, Dp, T, x2.dtype)
            else:
                eqlinear_bwd_x(dy2, _packed(w, EQL_PACK_BWDX), dx, N, Cp, Dp, T, x2.dtype)
            dx = dx.reshape(*ctx.lead_shape, Cp * T)
        if need_dw:
            dw = torch.empty_like(w)
            if train and need_dx:
                eqlinear_bwd_w_train(dy2, dw, ws, ctx.ws_bytes, N, Cp, Dp, T, x2.dtype)
            else:
                if ws is None:
                    ws = torch.empty(max(ctx.ws_bytes, 16), dtype=torch.uint8, device=x2.device)
                eqlinear_bwd_w(x2, dy2, dw, ws, ctx.ws_bytes, N, Cp, Dp, T, x2.dtype)
        return dx, dw, None


def eqlinear(x: torch.Tensor, w: torch.Tensor, keep_spectra: bool = True) -> torch.Tensor:
    """keep_spectra: with a weight gradient, run the training entry points (the forward keeps
    the weight-gradient workspace, about the size of x and dy plus fp32 partials, until the
    backward); False runs the plain passes and keeps only x."""
    return EQLinearFunction.apply(x, w, keep_spectra)


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
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, b, r, act, grad_mode: bool, keep_spectra: bool = True):
        Dp, Cp, T = w.shape
        if x.shape[-1] != Cp * T:
            raise ValueError("x has %d features, the weight expects C'*T = %d" % (x.shape[-1], Cp * T))
        if x.dtype != w.dtype or (b is not None and b.dtype != x.dtype) or (r is not None and r.dtype != x.dtype):
            raise ValueError("x, w, bias and residual must share a dtype (fp16 or fp32)")
        code = _act_code(act)
        # The kernel reads exactly D' bias values (one per output channel, shared by its
        # T group elements): a per-feature bias of D'*T values, or a short one, is refused.
        if b is not None and (b.dim() != 1 or b.numel() != Dp):
            raise ValueError("bias must be 1-D with D' = %d values (one per output channel, shared over the "
                             "group), got shape %s" % (Dp, tuple(b.shape)))
        if b is not None and b.device != x.device:
            raise ValueError("bias must be on x's device (%s), got %s" % (x.device, b.device))
        if r is not None and r.device != x.device:
            raise ValueError("residual must be on x's device (%s), got %s" % (x.device, r.device))
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
        bc = b.contiguous() if b is not None else None
        ws_bytes = eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, x.dtype)
        if keep_spectra and grad_mode and ctx.needs_input_grad[1]:
            # The weight gradient will follow: keep x's spectrum in its workspace.
            wsw = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
            eqlinear_fwd_fused_train(x2, _packed(w, EQL_PACK_FWD), bc, r2, y, pre, wsw, ws_bytes, N, Cp, Dp, T,
                                     x.dtype, code)
        else:
            wsw = None
            eqlinear_fwd_fused(x2, _packed(w, EQL_PACK_FWD), bc, r2, y, pre, N, Cp, Dp, T, x.dtype, code)
        ctx.save_for_backward(x2, w, pre, wsw)
        ctx.ws_bytes = ws_bytes
        ctx.code, ctx.has_bias, ctx.lead_shape = code, b is not None, x.shape[:-1]
        ctx.res_shape = r.shape if r is not None else None
        return y.reshape(*x.shape[:-1], Dp * T)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, w, pre, wsw = ctx.saved_tensors
        Dp, Cp, T = w.shape
        N = x2.shape[0]
        dy2 = dy.reshape(-1, Dp * T).to(x2.dtype).contiguous()
        dr = dy2.reshape(ctx.res_shape) if ctx.res_shape is not None and ctx.needs_input_grad[3] else None
        dx = dw = db = None
        if not any(ctx.needs_input_grad[:3]):
            return dx, dw, db, dr, None, None, None
        # Without an activation dpre = dy: the call then only sums the bias gradient.
        dpre = torch.empty_like(dy2) if ctx.code == EQL_ACT_GELU else dy2
        if ctx.has_bias and ctx.needs_input_grad[2]:
            db = torch.empty(Dp, dtype=x2.dtype, device=x2.device)
        if ctx.code == EQL_ACT_GELU or db is not None:
            ws_bytes = eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, x2.dtype)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x2.device)
            eqlinear_fused_epilogue_bwd(dy2, pre, dpre, db, ws, ws_bytes, N, Dp, T, x2.dtype, ctx.code)
        # With a weight gradient the training entry points run on dpre: the input gradient
        # leaves dpre's spectrum beside x's (from the forward) in the workspace.
        train = wsw is not None and ctx.needs_input_grad[1]
        if ctx.needs_input_grad[0]:
            dx = torch.empty((N, Cp * T), dtype=x2.dtype, device=x2.device)
            if train:
                eqlinear_bwd_x_train(dpre, _packed(w, EQL_PACK_BWDX), dx, wsw, ctx.ws_bytes, N, Cp, Dp, T, x2.dtype)
            else:
                eqlinear_bwd_x(dpre, _packed(w, EQL_PACK_BWDX), dx, N, Cp, Dp, T, x2.dtype)
            dx = dx.reshape(*ctx.lead_shape, Cp * T)
        if ctx.needs_input_grad[1]:
            dw = torch.empty_like(w)
            if train and ctx.needs_input_grad[0]:
                eqlinear_bwd_w_train(dpre, dw, wsw, ctx.ws_bytes, N, Cp, Dp, T, x2.dtype)
            else:
                wsb = wsw if wsw is not None else torch.empty(max(ctx.ws_bytes, 16), dtype=torch.uint8,
                                                              device=x2.device)
                eqlinear_bwd_w(x2, dpre, dw, wsb, ctx.ws_bytes, N, Cp, Dp, T, x2.dtype)
        return dx, dw, db, dr, None, None, None


def eqlinear_fused(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
                   residual: torch.Tensor | None = None, act: str = "none", keep_spectra: bool = True) -> torch.Tensor:
    """act(x W^T + bias) + residual with the epilogue fused into the forward kernel
    (eqlinear_fwd_fused), the MLP-block epilogue of the networks the layer is built into
    ("Nivel de Rede").  bias has one value per output channel (shared by its T group
    elements); act is "none" or "gelu"; residual has the output's shape.  Differentiable
    in x, w, bias and residual.  keep_spectra as for eqlinear."""
    return EQLinearFusedFunction.apply(x, w, bias, residual, act, torch.is_grad_enabled(), keep_spectra)


class EQLinear(torch.nn.Module):
    """Equivariant linear layer over C_T: in_channels*T -> out_channels*T features."""

    def __init__(self, in_channels: int, out_channels: int, group_order: int = 4, bias: bool = False,
                 activation: str | None = None, device=None, dtype=None, keep_spectra: bool = True):
        super().__init__()
        self.in_channels, self.out_channels, self.group_order = in_channels, out_channels, group_order
        # Training through the training entry points holds the weight-gradient workspace
        # from the forward to the backward (see eqlinear); False trades that memory for the
        # weight gradient's own transforms.
        self.keep_spectra = keep_spectra
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
            return EQLinearFunction.apply(x, self.weight, self.keep_spectra)
        return EQLinearFusedFunction.apply(x, self.weight, self.bias, residual, self.activation,
                                           torch.is_grad_enabled(), self.keep_spectra)

    def extra_repr(self) -> str:
        return "in_channels=%d, out_channels=%d, group_order=%d, bias=%s, activation=%s" % (
            self.in_channels, self.out_channels, self.group_order, self.bias is not None, self.activation)


class EQLinearP4MFunction(torch.autograd.Function):
    """The layer over p4m's point group (dihedral D4): y[..., D'*8] = x[..., C'*8] W^T with
    W[(d,g),(c,h)] = w[d, c, g h^-1], group axis r^0..r^3 then r^-m s (m = 0..3).  Run as the
    C_4 layer on 2C' x 2D' channels with the tied weight eqlinear_p4m_expand_weight builds;
    the weight gradient is the C_4 one folded back onto the shared parameters."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, keep_spectra: bool = True):
        Dp, Cp, G = w.shape
        if G != 8:
            raise ValueError("a p4m weight has 8 group elements per (out, in) pair, got %d" % G)
        if x.shape[-1] != Cp * 8:
            raise ValueError("x has %d features, the weight expects C'*8 = %d" % (x.shape[-1], Cp * 8))
        if x.dtype != w.dtype:
            raise ValueError("x and w must share a dtype (fp16 or fp32)")
        w4 = torch.empty((2 * Dp, 2 * Cp, 4), dtype=w.dtype, device=w.device)
        eqlinear_p4m_expand_weight(w.contiguous(), w4, Dp, Cp, w.dtype)
        x2 = x.reshape(-1, Cp * 8).contiguous()
        N = x2.shape[0]
        y = torch.empty((N, Dp * 8), dtype=x.dtype, device=x.device)
        ws_bytes = eqlinear_bwd_w_workspace_bytes(N, 2 * Cp, 2 * Dp, 4, x.dtype)
        if keep_spectra and ctx.needs_input_grad[1]:
            # As EQLinearFunction: keep x's spectrum for the weight gradient.
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
            eqlinear_fwd_train(x2, _packed(w4, EQL_PACK_FWD), y, ws, ws_bytes, N, 2 * Cp, 2 * Dp, 4, x.dtype)
        else:
            ws = None
            eqlinear_fwd(x2, _packed(w4, EQL_PACK_FWD), y, N, 2 * Cp, 2 * Dp, 4, x.dtype)
        ctx.save_for_backward(x2, w4, ws)
        ctx.ws_bytes = ws_bytes
        ctx.lead_shape = x.shape[:-1]
        ctx.p4m_shape = (Dp, Cp)
        return y.reshape(*x.shape[:-1], Dp * 8)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, w4, ws = ctx.saved_tensors
        Dp, Cp = ctx.p4m_shape
        N = x2.shape[0]
        dy2 = dy.reshape(-1, Dp * 8).to(x2.dtype).contiguous()
        dx = dw = None
        need_dx, need_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        train = ws is not None
        if need_dx:
            dx = torch.empty((N, Cp * 8), dtype=x2.dtype, device=x2.device)
            if train and need_dw:
                eqlinear_bwd_x_train(dy2, _packed(w4, EQL_PACK_BWDX), dx, ws, ctx.ws_bytes, N, 2 * Cp, 2 * Dp, 4,
                                     x2.dtype)
            else:
                eqlinear_bwd_x(dy2, _packed(w4, EQL_PACK_BWDX), dx, N, 2 * Cp, 2 * Dp, 4, x2.dtype)
            dx = dx.reshape(*ctx.lead_shape, Cp * 8)
        if need_dw:
            dw4 = torch.empty_like(w4)
            if train and need_dx:
                eqlinear_bwd_w_train(dy2, dw4, ws, ctx.ws_bytes, N, 2 * Cp, 2 * Dp, 4, x2.dtype)
            else:
                if ws is None:
                    ws = torch.empty(max(ctx.ws_bytes, 16), dtype=torch.uint8, device=x2.device)
                eqlinear_bwd_w(x2, dy2, dw4, ws, ctx.ws_bytes, N, 2 * Cp, 2 * Dp, 4, x2.dtype)
            dw = torch.empty((Dp, Cp, 8), dtype=x2.dtype, device=x2.device)
            eqlinear_p4m_fold_weight_grad(dw4, dw, Dp, Cp, x2.dtype)
        return dx, dw, None


def eqlinear_p4m(x: torch.Tensor, w: torch.Tensor, keep_spectra: bool = True) -> torch.Tensor:
    """keep_spectra as for eqlinear."""
    return EQLinearP4MFunction.apply(x, w, keep_spectra)


class EQLinearP4M(torch.nn.Module):
    """Equivariant linear layer over p4m's point group: in_channels*8 -> out_channels*8."""

    def __init__(self, in_channels: int, out_channels: int, device=None, dtype=None, keep_spectra: bool = True):
        super().__init__()
        self.in_channels, self.out_channels = in_channels, out_channels
        self.keep_spectra = keep_spectra
        self.weight = torch.nn.Parameter(torch.empty(out_channels, in_channels, 8, device=device, dtype=dtype))
        with torch.no_grad():
            self.weight.normal_(0.0, 1.0 / math.sqrt(in_channels * 8))

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return EQLinearP4MFunction.apply(x, self.weight, self.keep_spectra)

    def extra_repr(self) -> str:
        return "in_channels=%d, out_channels=%d, group=p4m" % (self.in_channels, self.out_channels)

