"""The linear layer fused with the cross-entropy: PyTorch-facing API over
ce_linear_forward (include/ce.h).

``linear_cross_entropy(hidden, weight, target, ...)`` is
``cross_entropy(hidden @ weight.T, target, ...)`` with the options of the
Liger-Kernel page "Kernel Profile: CrossEntropy (Tier 3 - Fused/Complex)"
(Forward Pass, Module Parameters), computed in row chunks (at most 2048 rows
by default), so a batch of more rows never holds its full (rows, V) logits
at once (the page's Classification names the fused linear cross-entropy as
this kernel extended with the linear layer).

Gradients: for reduction "mean" and "sum" the forward computes
d loss / d hidden and d loss / d weight with the loss (gradient in forward);
the backward scales them by grad_output with the library's scaling kernel.
For "none" the per-row grad_output is known only in the backward, which
then calls the library again with it.

PyTorch supplies memory and the stream; every step runs in the library.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import CE_BF16, CE_F32, REDUCTION_CODES, check
from .functional import CEOutput, _stream


def _ptr(a: Optional[torch.Tensor]) -> int:
    return 0 if a is None else a.data_ptr()


def linear_forward_raw(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                       class_weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                       label_smoothing: float = 0.0, lse_square_scale: float = 0.0,
                       softcap: Optional[float] = None, reduction: str = "mean",
                       grad: bool = True, grad_output: Optional[torch.Tensor] = None,
                       z_loss: bool = False, token_accuracy: bool = False,
                       argmax: bool = False, counts: bool = False, chunk_rows: int = 0,
                       flags: int = 0):
    """One ce_linear_forward call. hidden (rows, H) and weight (V, H) bf16 on
    the GPU. Returns (loss, z_loss, token_accuracy, argmax, counts,
    grad_hidden, grad_weight); the gradients are fp32 (or None)."""
    if not (hidden.is_cuda and weight.is_cuda):
        raise ValueError("hidden and weight must be CUDA (HIP) tensors")
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError("hidden must be (rows, H) and weight (V, H)")
    if hidden.stride(1) != 1:
        hidden = hidden.contiguous()
    if weight.stride(1) != 1:
        weight = weight.contiguous()
    if reduction not in REDUCTION_CODES:
        raise ValueError(f"reduction must be one of {tuple(REDUCTION_CODES)}")
    dev = hidden.device
    rows, H = hidden.shape
    V = weight.shape[0]
    t = target.reshape(-1).to(device=dev, dtype=torch.int64).contiguous()
    if t.numel() != rows:
        raise ValueError("target must have one entry per row of hidden")
    cw = None
    if class_weight is not None:
        cw = class_weight.to(device=dev, dtype=torch.float32).contiguous()
    f32 = dict(device=dev, dtype=torch.float32)
    shape = (rows,) if reduction == "none" else ()
    loss = torch.empty(shape, **f32)
    zl = torch.empty(shape, **f32) if z_loss else None
    acc = torch.empty(shape, **f32) if token_accuracy else None
    am = torch.empty((rows,), device=dev, dtype=torch.int64) if argmax else None
    cnt = torch.empty((2,), device=dev, dtype=torch.int64) if counts else None
    gh = torch.empty((rows, H), **f32) if grad else None
    gw = torch.empty((V, H), **f32) if grad else None
    per_row = 0
    go = None
    if grad_output is not None:
        go = grad_output.to(device=dev, dtype=torch.float32).contiguous()
        per_row = 1 if go.numel() == rows and reduction == "none" and go.dim() > 0 else 0
    nbytes = _lib.ce_linear_workspace_bytes(rows, H, V, chunk_rows, flags)
    if nbytes == 0:
        raise ValueError(f"invalid sizes rows={rows} H={H} V={V} chunk_rows={chunk_rows}")
    # Allocated per call (returned to torch's caching allocator afterwards,
    # not held by this module): the library clears what it needs itself.
    ws = torch.empty((nbytes,), device=dev, dtype=torch.uint8)
    st = _lib.ce_linear_forward(
        hidden.data_ptr(), hidden.stride(0), weight.data_ptr(), weight.stride(0), CE_BF16, rows,
        H, V, t.data_ptr(), _ptr(cw), ignore_index, label_smoothing, lse_square_scale,
        float(softcap) if softcap else 0.0, REDUCTION_CODES[reduction], flags, _ptr(go), per_row,
        chunk_rows, loss.data_ptr(), _ptr(zl), _ptr(acc), _ptr(am), _ptr(cnt), _ptr(gh), H,
        _ptr(gw), H, ws.data_ptr(), nbytes, _stream(dev))
    check(st, "ce_linear_forward")
    return loss, zl, acc, am, cnt, gh, gw


class LinearCrossEntropyFunction(torch.autograd.Function):
    """Autograd over ce_linear_forward (gradients of hidden and weight)."""

    @staticmethod
    def forward(ctx, hidden, weight, target, class_weight, ignore_index, lse_square_scale,
                label_smoothing, reduction, softcap, want_z, want_acc, want_arg, chunk_rows):
        need = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
        in_forward = need and reduction != "none"
        loss, zl, acc, am, _, gh, gw = linear_forward_raw(
            hidden, weight, target, class_weight, ignore_index, label_smoothing,
            lse_square_scale, softcap, reduction, grad=in_forward, z_loss=want_z,
            token_accuracy=want_acc, argmax=want_arg, chunk_rows=chunk_rows)
        ctx.in_forward = in_forward
        ctx.opts = (ignore_index, label_smoothing, lse_square_scale, softcap, reduction,
                    chunk_rows)
        if in_forward:
            ctx.save_for_backward(gh, gw)
        elif need:
            ctx.save_for_backward(hidden, weight, target, class_weight)
        for o in (zl, acc, am):
            if o is not None:
                ctx.mark_non_differentiable(o)
        return loss, zl, acc, am

    @staticmethod
    def backward(ctx, grad_loss, *_):
        if ctx.in_forward:
            gh, gw = ctx.saved_tensors
            go = grad_loss.to(torch.float32).reshape(())
            st = _stream(gh.device)
            # grad_output == 1 leaves them untouched (the kernel exits at once)
            for g in (gh, gw):
                check(_lib.ce_backward(g.data_ptr(), CE_F32, g.shape[0], g.shape[1], g.shape[1],
                                       go.data_ptr(), 0, st), "ce_backward")
        else:
            hidden, weight, target, class_weight = ctx.saved_tensors
            ig, eps, lam, sc, red, chunk = ctx.opts
            _, _, _, _, _, gh, gw = linear_forward_raw(
                hidden, weight, target, class_weight, ig, eps, lam, sc, red, grad=True,
                grad_output=grad_loss, chunk_rows=chunk)
        return gh, gw, None, None, None, None, None, None, None, None, None, None, None


def linear_cross_entropy(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                         class_weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                         lse_square_scale: float = 0.0, label_smoothing: float = 0.0,
                         reduction: str = "mean", softcap: Optional[float] = None,
                         return_z_loss: bool = False, return_token_accuracy: bool = False,
                         return_predicted_tokens: bool = False,
                         chunk_rows: int = 0) -> CEOutput:
    """cross_entropy(hidden @ weight.T, target) without holding the (rows, V)
    logits at once. hidden (..., H) and weight (V, H) are bfloat16; the
    returned loss, z_loss and token_accuracy are fp32."""
    H = hidden.shape[-1]
    h2 = hidden.reshape(-1, H)
    t = target.reshape(-1)
    loss, zl, acc, am = LinearCrossEntropyFunction.apply(
        h2, weight, t, class_weight, ignore_index, lse_square_scale, label_smoothing, reduction,
        softcap, return_z_loss, return_token_accuracy, return_predicted_tokens, chunk_rows)
    if reduction == "none":
        shape = tuple(hidden.shape[:-1])
        loss = loss.reshape(shape)
        zl = zl.reshape(shape) if zl is not None else None
        acc = acc.reshape(shape) if acc is not None else None
    if am is not None:
        am = am.reshape(tuple(hidden.shape[:-1]))
    return CEOutput(loss, zl, acc, am)


class LinearCrossEntropyLoss(torch.nn.Module):
    """Module form of linear_cross_entropy (the layer's weight is passed to
    forward, as a language-model head's weight usually is)."""

    def __init__(self, class_weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                 lse_square_scale: float = 0.0, label_smoothing: float = 0.0,
                 reduction: str = "mean", softcap: Optional[float] = None,
                 return_z_loss: bool = False, chunk_rows: int = 0):
        super().__init__()
        self.class_weight = class_weight
        self.ignore_index = ignore_index
        self.lse_square_scale = lse_square_scale
        self.label_smoothing = label_smoothing
        self.reduction = reduction
        self.softcap = softcap
        self.return_z_loss = return_z_loss
        self.chunk_rows = chunk_rows

    def forward(self, hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor):
        out = linear_cross_entropy(hidden, weight, target, self.class_weight, self.ignore_index,
                                   self.lse_square_scale, self.label_smoothing, self.reduction,
                                   self.softcap, self.return_z_loss, chunk_rows=self.chunk_rows)
        return (out.loss, out.z_loss) if self.return_z_loss else out.loss
