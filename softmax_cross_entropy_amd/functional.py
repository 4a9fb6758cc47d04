"""PyTorch-facing API over the C ABI: a functional, an autograd Function and
a loss module, with the parameters and defaults of the Liger-Kernel page
"Kernel Profile: CrossEntropy (Tier 3 - Fused/Complex)" (Forward Pass and
Module Parameters).

PyTorch supplies device memory and the stream; every computation runs in
the HIP kernels behind the C ABI.

Gradient-in-forward (the page's Key Patterns): when the logits require a
gradient, the forward overwrites their storage with d loss / d logits and
the backward rescales that buffer by grad_output in place. The logits tensor
passed in must therefore not be used again after the call; pass
``inplace=False`` to work on a private copy instead, or ``keep_logits=True``
to leave the logits untouched and recompute the gradient in the backward from
the logits and the per-row (max, log-sum) the forward keeps (the saved-logits
backward of the tt-mlir PR #9324 page's cross_entropy_bw composite).
"""

from __future__ import annotations

from collections import namedtuple
from typing import Optional

import torch

from . import _lib
from ._lib import (CE_F_CHECK_TARGETS, CE_F_GRAD, REDUCTION_CODES, check, dtype_code)

CEOutput = namedtuple("CEOutput", ["loss", "z_loss", "token_accuracy", "predicted_tokens"])


def _flatten(logits: torch.Tensor, target: torch.Tensor):
    """(..., V) class-last logits -> a 2-D (rows, V) view with unit class stride.

    Rank-1 inputs are rejected (the PR #9324 page tests a rank-1 rejection).
    """
    if logits.dim() < 2:
        raise ValueError("logits must have at least 2 dimensions (..., V); got rank "
                         f"{logits.dim()}")
    V = logits.shape[-1]
    if tuple(target.shape) != tuple(logits.shape[:-1]):
        raise ValueError(f"target shape {tuple(target.shape)} must equal logits.shape[:-1] "
                         f"{tuple(logits.shape[:-1])}")
    x2 = logits.reshape(-1, V) if logits.dim() != 2 else logits
    if x2.stride(-1) != 1 or (x2.shape[0] > 1 and x2.stride(0) < V):
        x2 = x2.contiguous()
    return x2, target.reshape(-1)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


_WORKSPACES = {}


def release_workspaces() -> None:
    """Drop the cached workspaces of every device and stream (the next call
    allocates and clears a new one)."""
    _WORKSPACES.clear()


def _workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    """Zero-filled workspace cached per (device, stream), grown on demand.

    The library leaves a workspace reusable after every call, so it is
    cleared only when it is first allocated.
    """
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), _stream(dev))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros((max(nbytes, 1 << 16),), device=dev, dtype=torch.uint8)
        _WORKSPACES[key] = ws
    return ws


def _forward_raw(x2: torch.Tensor, t: torch.Tensor, weight: Optional[torch.Tensor],
                 ignore_index: int, label_smoothing: float, lse_square_scale: float,
                 softcap: Optional[float], reduction: str, want_grad: bool,
                 want_z: bool, want_acc: bool, want_arg: bool, want_counts: bool = False,
                 check_targets: bool = False, extra_flags: int = 0,
                 row_stats: Optional[torch.Tensor] = None):
    if not x2.is_cuda:
        raise ValueError("logits must be a CUDA (HIP) tensor")
    if reduction not in REDUCTION_CODES:
        raise ValueError(f"reduction must be one of {tuple(REDUCTION_CODES)}")
    dev = x2.device
    dt = dtype_code(x2.dtype)
    rows, V = x2.shape
    t = t.to(device=dev, dtype=torch.int64).contiguous()
    w = None
    if weight is not None:
        w = weight.to(device=dev, dtype=torch.float32).contiguous()
        if w.shape != (V,):
            raise ValueError(f"weight must have shape ({V},)")
    flags = extra_flags | (CE_F_GRAD if want_grad else 0) | (CE_F_CHECK_TARGETS if check_targets else 0)
    red = REDUCTION_CODES[reduction]
    out_shape = (rows,) if reduction == "none" else ()
    f32 = dict(device=dev, dtype=torch.float32)
    loss = torch.empty(out_shape, **f32)
    z_loss = torch.empty(out_shape, **f32) if want_z else None
    acc = torch.empty(out_shape, **f32) if want_acc else None
    arg = torch.empty((rows,), device=dev, dtype=torch.int64) if want_arg else None
    counts = torch.empty((2,), device=dev, dtype=torch.int64) if want_counts else None
    ws_bytes = _lib.ce_workspace_bytes(rows, V, dt, flags)
    if ws_bytes == 0:
        raise ValueError("invalid problem size")
    ws = _workspace(dev, ws_bytes)

    def ptr(a):
        return 0 if a is None else a.data_ptr()

    status = _lib.ce_forward(ptr(x2), dt, rows, V, x2.stride(0) if rows > 0 else V, ptr(t),
                             ptr(w), int(ignore_index), float(label_smoothing),
                             float(lse_square_scale), float(softcap or 0.0), red, flags,
                             ptr(loss), ptr(z_loss), ptr(acc), ptr(arg), ptr(counts),
                             ptr(row_stats), ptr(ws), ws_bytes, _stream(dev))
    check(status, "ce_forward")
    return loss, z_loss, acc, arg, counts


def backward_recompute(x2: torch.Tensor, t: torch.Tensor, weight: Optional[torch.Tensor],
                       ignore_index: int, label_smoothing: float, lse_square_scale: float,
                       softcap: Optional[float], reduction: str, row_stats: torch.Tensor,
                       grad_output: torch.Tensor, grad: Optional[torch.Tensor] = None
                       ) -> torch.Tensor:
    """grad (rows, V) = grad_output * d loss / d logits, recomputed from the kept
    logits x2 and the forward's row_stats; a new tensor unless ``grad`` is given
    (which may be x2 itself)."""
    dev = x2.device
    dt = dtype_code(x2.dtype)
    rows, V = x2.shape
    _check_grad_output(grad_output, rows, reduction == "none")
    if grad is None:
        grad = torch.empty((rows, V), device=dev, dtype=x2.dtype)
    t = t.to(device=dev, dtype=torch.int64).contiguous()
    w = None if weight is None else weight.to(device=dev, dtype=torch.float32).contiguous()
    go = grad_output.to(device=dev, dtype=torch.float32).contiguous().reshape(-1)
    ws = _workspace(dev, 256)
    status = _lib.ce_backward_recompute(
        x2.data_ptr(), dt, rows, V, x2.stride(0) if rows > 0 else V, t.data_ptr(),
        0 if w is None else w.data_ptr(), int(ignore_index), float(label_smoothing),
        float(lse_square_scale), float(softcap or 0.0), REDUCTION_CODES[reduction],
        row_stats.data_ptr(), go.data_ptr(), 1 if reduction == "none" else 0, grad.data_ptr(),
        grad.stride(0) if rows > 0 else V, ws.data_ptr(), ws.numel(), _stream(dev))
    check(status, "ce_backward_recompute")
    return grad


def _check_grad_output(grad_output: torch.Tensor, rows: int, per_row: bool) -> None:
    """The kernels read one grad_output value, or one per row: any other
    length is an error here, not a read past the tensor."""
    want = rows if per_row else 1
    if grad_output.numel() != want:
        raise ValueError(f"grad_output must hold {want} value(s) "
                         f"({'one per row' if per_row else 'a scalar'}), got {grad_output.numel()}")


def backward_(grad2: torch.Tensor, grad_output: torch.Tensor, per_row: bool) -> torch.Tensor:
    """In place: grad2 (rows, V) *= grad_output (scalar, or per row)."""
    rows, V = grad2.shape
    _check_grad_output(grad_output, rows, per_row)
    go = grad_output.to(device=grad2.device, dtype=torch.float32).contiguous().reshape(-1)
    status = _lib.ce_backward(grad2.data_ptr(), dtype_code(grad2.dtype), rows, V,
                              grad2.stride(0) if rows > 0 else V, go.data_ptr(),
                              1 if per_row else 0, _stream(grad2.device))
    check(status, "ce_backward")
    return grad2


class CrossEntropyFunction(torch.autograd.Function):
    """Fused forward (+ gradient into the logits' storage) and a scaling backward."""

    @staticmethod
    def forward(ctx, logits, target, weight, ignore_index, lse_square_scale, label_smoothing,
                reduction, softcap, return_z_loss, return_token_accuracy,
                return_predicted_tokens, inplace, keep_logits=False):
        want_grad = logits.requires_grad
        x2, t = _flatten(logits, target)
        work = x2.detach()
        if want_grad and not inplace and not keep_logits:
            work = work.clone()
        stats = None
        if want_grad and keep_logits:
            stats = torch.empty((x2.shape[0], 2), device=x2.device, dtype=torch.float32)
        loss, z_loss, acc, arg, _ = _forward_raw(
            work, t, weight, ignore_index, label_smoothing, lse_square_scale, softcap,
            reduction, want_grad and not keep_logits, return_z_loss, return_token_accuracy,
            return_predicted_tokens, row_stats=stats)
        lead = logits.shape[:-1]
        if reduction == "none":
            loss = loss.reshape(lead)
            z_loss = z_loss.reshape(lead) if z_loss is not None else None
            acc = acc.reshape(lead) if acc is not None else None
        if arg is not None:
            arg = arg.reshape(lead)
        ctx.reduction = reduction
        ctx.shape = logits.shape
        ctx.keep_logits = keep_logits
        if want_grad and keep_logits:
            ctx.options = (ignore_index, label_smoothing, lse_square_scale, softcap)
            ctx.save_for_backward(work, t, stats, weight)
        elif want_grad:
            ctx.save_for_backward(work)
        for o in (z_loss, acc, arg):
            if o is not None:
                ctx.mark_non_differentiable(o)
        return loss, z_loss, acc, arg

    @staticmethod
    def backward(ctx, grad_loss, *_):
        if ctx.keep_logits:
            x2, t, stats, weight = ctx.saved_tensors
            ii, eps, lam, cap = ctx.options
            g = backward_recompute(x2, t, weight, ii, eps, lam, cap, ctx.reduction, stats,
                                   grad_loss)
        else:
            (g,) = ctx.saved_tensors
            backward_(g, grad_loss, per_row=(ctx.reduction == "none"))
        return (g.view(ctx.shape),) + (None,) * 12


def cross_entropy(logits: torch.Tensor, target: torch.Tensor, weight: Optional[torch.Tensor] = None,
                  ignore_index: int = -100, lse_square_scale: float = 0.0,
                  label_smoothing: float = 0.0, reduction: str = "mean",
                  softcap: Optional[float] = None, return_z_loss: bool = False,
                  return_token_accuracy: bool = False, return_predicted_tokens: bool = False,
                  inplace: bool = True, keep_logits: bool = False):
    """Fused softmax cross-entropy. Returns the loss, or a CEOutput when any
    ``return_*`` flag is set (fields not requested are None). ``keep_logits``:
    the logits are left intact and the backward recomputes the gradient."""
    if softcap is not None and softcap <= 0:
        raise ValueError("softcap must be None or > 0")
    loss, z, acc, arg = CrossEntropyFunction.apply(
        logits, target, weight, ignore_index, lse_square_scale, label_smoothing, reduction,
        softcap, return_z_loss, return_token_accuracy, return_predicted_tokens, inplace,
        keep_logits)
    if return_z_loss or return_token_accuracy or return_predicted_tokens:
        return CEOutput(loss, z, acc, arg)
    return loss


class CrossEntropyLoss(torch.nn.Module):
    """Module form; no learnable parameters."""

    def __init__(self, weight: Optional[torch.Tensor] = None, ignore_index: int = -100,
                 lse_square_scale: float = 0.0, label_smoothing: float = 0.0,
                 reduction: str = "mean", softcap: Optional[float] = None,
                 return_z_loss: bool = False, return_token_accuracy: bool = False,
                 return_predicted_tokens: bool = False, inplace: bool = True,
                 keep_logits: bool = False):
        super().__init__()
        if reduction not in REDUCTION_CODES:
            raise ValueError(f"reduction must be one of {tuple(REDUCTION_CODES)}")
        if not 0.0 <= label_smoothing <= 1.0:
            raise ValueError("label_smoothing must be in [0, 1]")
        if softcap is not None and softcap <= 0:
            raise ValueError("softcap must be None or > 0")
        self.register_buffer("weight", weight, persistent=False)
        self.ignore_index = ignore_index
        self.lse_square_scale = lse_square_scale
        self.label_smoothing = label_smoothing
        self.reduction = reduction
        self.softcap = softcap
        self.return_z_loss = return_z_loss
        self.return_token_accuracy = return_token_accuracy
        self.return_predicted_tokens = return_predicted_tokens
        self.inplace = inplace
        self.keep_logits = keep_logits

    def forward(self, logits: torch.Tensor, target: torch.Tensor):
        return cross_entropy(logits, target, self.weight, self.ignore_index,
                             self.lse_square_scale, self.label_smoothing, self.reduction,
                             self.softcap, self.return_z_loss, self.return_token_accuracy,
                             self.return_predicted_tokens, self.inplace, self.keep_logits)


def forward_raw(logits2d: torch.Tensor, target: torch.Tensor, weight=None, ignore_index=-100,
                label_smoothing=0.0, lse_square_scale=0.0, softcap=None, reduction="mean",
                grad=True, z_loss=False, token_accuracy=False, argmax=False, counts=False,
                check_targets=False, flags=0, row_stats=None):
    """Direct call of ce_forward on a 2-D (rows, V) tensor (overwritten by the
    gradient when ``grad``). Returns (loss, z_loss, token_accuracy, argmax, counts);
    ``row_stats``, a (rows, 2) float32 tensor, receives the per-row (m, log2 s)."""
    if logits2d.dim() != 2 or logits2d.stride(-1) != 1:
        raise ValueError("logits2d must be 2-D with unit class stride")
    return _forward_raw(logits2d, target, weight, ignore_index, label_smoothing,
                        lse_square_scale, softcap, reduction, grad, z_loss, token_accuracy,
                        argmax, counts, check_targets, flags, row_stats)
