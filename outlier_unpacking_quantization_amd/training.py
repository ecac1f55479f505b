"""Quantized-training linear layer: y = x W^T, whose three GEMMs per step
(forward, data gradient, weight gradient) each run the whole IM-Unpack path
through ``imu_imunpack_matmul``.

Method: summary page "IM-Unpack: Training and Inference with Arbitrarily Low
Precision Integers", summary paragraph and "Key results": the page trains
models with the GEMMs of the forward and the backward pass replaced by their
low bit-width integer versions, which IM-Unpack computes exactly from the RTN
codes of the operands (no clipping of heavy hitters).  Each product below is
one such GEMM:

    forward          y  = x  @ W^T     A = x  (tokens x d_in),   B = W^T
    data gradient    dx = dy @ W       A = dy (tokens x d_out),  B = W
    weight gradient  dW = dy^T @ x     A = dy^T,                 B = x

Every operand is quantized once per matrix, whatever the product it enters
(its own percentile scale, shared by every use): X and W in the forward, dY in
the backward, three quantization passes per step instead of one per operand
per product.  Each prepared tensor carries the statistics of both line
directions, so a GEMM that uses it transposed (W^T in the forward, dY^T in the
weight gradient) swaps their roles; unpacking plans stay per product.
Transposes are views (no copies), and the incoming gradient enters as float32,
so no rounding happens before its RTN.  The outputs are the dequantized
float32 products; autograd receives them in the dtype of the tensor they
belong to.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import binding as B


def prepare(t: torch.Tensor, p: B.ImuParams) -> B.Stats:
    """Quantization statistics of a (rows, cols) tensor for every product it enters."""
    return B.prepare_operand(B.Matrix(t), p)


def linear_forward(x: torch.Tensor, w: torch.Tensor, p: B.ImuParams, ws: Optional[B.Workspace] = None,
                   sx: Optional[B.Stats] = None, sw: Optional[B.Stats] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(y float32, C int32) of y = x @ W^T; x: (tokens, d_in), w: (d_out, d_in).
    sx / sw: statistics from prepare() (computed in the call when None)."""
    out, c, _ = B.imunpack_matmul_prepared(B.Matrix(x), B.Matrix(w, "transposed"), p, sx,
                                           (sw, True) if sw is not None else None, ws=ws)
    return out[0], c[0]


def linear_data_grad(dy: torch.Tensor, w: torch.Tensor, p: B.ImuParams, ws: Optional[B.Workspace] = None,
                     sdy: Optional[B.Stats] = None, sw: Optional[B.Stats] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(dx float32, C int32) of dx = dy @ W; dy: (tokens, d_out), w: (d_out, d_in)."""
    out, c, _ = B.imunpack_matmul_prepared(B.Matrix(dy), B.Matrix(w), p, sdy, sw, ws=ws)
    return out[0], c[0]


def linear_weight_grad(dy: torch.Tensor, x: torch.Tensor, p: B.ImuParams, ws: Optional[B.Workspace] = None,
                       sdy: Optional[B.Stats] = None, sx: Optional[B.Stats] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(dW float32, C int32) of dW = dy^T @ x; dy: (tokens, d_out), x: (tokens, d_in)."""
    out, c, _ = B.imunpack_matmul_prepared(B.Matrix(dy, "transposed"), B.Matrix(x), p,
                                           (sdy, True) if sdy is not None else None, sx, ws=ws)
    return out[0], c[0]


def training_step(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, p: B.ImuParams,
                  ws: Optional[B.Workspace] = None):
    """The three products of a training step with each operand quantized once:
    returns ((y, C_y), (dx, C_dx), (dW, C_dW))."""
    sx, sw, sdy = prepare(x, p), prepare(w, p), prepare(dy, p)
    return (linear_forward(x, w, p, ws, sx, sw), linear_data_grad(dy, w, p, ws, sdy, sw),
            linear_weight_grad(dy, x, p, ws, sdy, sx))


class IMUnpackLinearFunction(torch.autograd.Function):
    """y = x @ W^T with the forward and both gradients computed by IM-Unpack."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, p: B.ImuParams, ws: Optional[B.Workspace]):
        if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
            raise B.ImunpackError(B.ERR_INVALID_ARG, "x must be (tokens, d_in) and w (d_out, d_in)")
        x, w = x.contiguous(), w.contiguous()
        sx, sw = prepare(x, p), prepare(w, p)  # each reused by a gradient GEMM
        ctx.save_for_backward(x, w)
        ctx.p, ctx.ws, ctx.sx, ctx.sw = p, ws, sx, sw
        return linear_forward(x, w, p, ws, sx, sw)[0]

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, w = ctx.saved_tensors
        dy = dy.to(torch.float32).contiguous()
        sdy = prepare(dy, ctx.p)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = linear_data_grad(dy, w, ctx.p, ctx.ws, sdy, ctx.sw)[0].to(x.dtype)
        if ctx.needs_input_grad[1]:
            dw = linear_weight_grad(dy, x, ctx.p, ctx.ws, sdy, ctx.sx)[0].to(w.dtype)
        ctx.sx = ctx.sw = None
        return dx, dw, None, None


def imunpack_linear(x: torch.Tensor, w: torch.Tensor, p: B.ImuParams,
                    ws: Optional[B.Workspace] = None) -> torch.Tensor:
    """y = x @ W^T (float32) with IM-Unpack in the forward and the backward pass."""
    return IMUnpackLinearFunction.apply(x, w, p, ws)
