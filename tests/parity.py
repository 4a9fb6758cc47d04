"""Parity helpers: run the HIP path and the float64 oracle on the same inputs
and compare them to the bar the tests state.

Tolerances (written here once, used by every GPU parity test):
  * loss, z_loss (scalars and per-row "none" values): relative 1e-5; an
    oracle value of exactly 0 must be exactly 0 on the GPU; NaN must match.
  * fp32 gradients: absolute 2e-6.
  * bf16 gradients: |g - G*| <= ulp_bf16(G*) + 2**-20 * M + 2**-126, where
    G* is the unrounded float64 gradient, ulp_bf16 the bf16 spacing at |G*|,
    M the sum of the magnitudes of the gradient's terms (cancellation scale)
    and 2**-126 the float32 underflow threshold.
  * argmax, counts, token_accuracy (bits of the float32 value): exact.
  * gradients of rows that are not counted: exactly +0.0.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import reduce_rows, rows_forward, summarize_targets

LOSS_RTOL = 1e-5
F32_GRAD_ATOL = 2e-6
BF16_FLOOR = 2.0 ** -20
F32_TINY = 2.0 ** -126


def host_logits(x: torch.Tensor) -> np.ndarray:
    """Host copy the oracle reads: float32 as is, bf16 as raw bit patterns."""
    x = x.detach().cpu()
    if x.dtype == torch.bfloat16:
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def assert_loss_close(gpu, want, what="loss"):
    g = np.asarray(gpu, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    nan_w = np.isnan(w)
    assert np.array_equal(np.isnan(g), nan_w), f"{what}: NaN pattern differs"
    zero = (w == 0.0)
    assert np.all(g[zero] == 0.0), f"{what}: oracle zeros not exactly zero on the GPU"
    m = ~nan_w & ~zero
    if m.any():
        rel = np.abs(g[m] - w[m]) / np.abs(w[m])
        i = int(np.argmax(rel))
        assert rel.max() <= LOSS_RTOL, (
            f"{what}: max rel err {rel.max():.3e} at {i}: gpu {g[m][i]!r} oracle {w[m][i]!r}")


def assert_grad_close(gpu: torch.Tensor, want: np.ndarray, mag: np.ndarray, zero_rows=None,
                      what="grad"):
    """zero_rows: boolean mask of rows (not counted) whose gradient must be +0.0."""
    dt = gpu.dtype
    g = gpu.detach().float().cpu().double().numpy()
    assert g.shape == want.shape
    if zero_rows is not None and np.any(zero_rows):
        gz = g[np.asarray(zero_rows)]
        bad0 = (gz != 0.0) | np.signbit(gz)
        assert not bad0.any(), f"{what}: {int(bad0.sum())} elements of rows that are not counted are not +0.0"
    err = np.abs(g - want)
    if dt == torch.float32:
        tol = np.full_like(want, F32_GRAD_ATOL)
    else:
        tol = bf16_ulp(want) + BF16_FLOOR * mag + F32_TINY
    over = err > tol
    if over.any():
        i = np.unravel_index(int(np.argmax(err - tol)), err.shape)
        raise AssertionError(
            f"{what}: {int(over.sum())} elements over tolerance; worst at {i}: gpu {g[i]!r} "
            f"oracle {want[i]!r} tol {tol[i]:.3e}")


class OracleRef:
    """Oracle results for a batch (optionally only for a sample of rows)."""

    def __init__(self, x_host, t_host, *, weight=None, ignore_index=-100, label_smoothing=0.0,
                 lse_square_scale=0.0, softcap=None, reduction="mean", rows=None,
                 want_grad=True, chunk=128):
        V = x_host.shape[1]
        w = None if weight is None else np.asarray(weight, dtype=np.float64)
        t = np.asarray(t_host, dtype=np.int64)
        self.summ = summarize_targets(t, V, ignore_index, w, reduction)
        sel = np.arange(t.shape[0]) if rows is None else np.asarray(rows)
        self.rows = sel
        self.not_counted = ~self.summ.counted[sel]
        n = sel.shape[0]
        self.ce = np.zeros(n)
        self.zeta = np.zeros(n)
        self.argmax = np.zeros(n, dtype=np.int64)
        self.correct = np.zeros(n, dtype=bool)
        self.grad = np.zeros((n, V)) if want_grad else None
        self.mag = np.zeros((n, V)) if want_grad else None
        for a in range(0, n, chunk):
            b = min(n, a + chunk)
            r = rows_forward(x_host[sel[a:b]], t[sel[a:b]], V=V, alpha=self.summ.alpha,
                             beta=self.summ.beta, weight=w, ignore_index=ignore_index,
                             label_smoothing=label_smoothing, lse_square_scale=lse_square_scale,
                             softcap=softcap, want_grad=want_grad, want_mag=want_grad)
            self.ce[a:b] = r.ce
            self.zeta[a:b] = r.zeta
            self.argmax[a:b] = r.argmax
            self.correct[a:b] = r.correct
            if want_grad:
                self.grad[a:b] = r.grad
                self.mag[a:b] = r.mag
        self.reduction = reduction
        if rows is None:
            self.loss, self.z_loss, self.acc, self.n_correct = reduce_rows(
                self.ce, self.zeta, self.correct, self.summ.counted, self.summ.n, self.summ.D,
                reduction)


def f32_bits(v) -> int:
    return int(np.array(v, dtype=np.float32).view(np.uint32))


def assert_acc_exact(gpu_val, n_correct, n):
    want = np.float64(n_correct) / np.float64(n) if n else math.nan
    if math.isnan(want):
        assert math.isnan(float(gpu_val))
    else:
        assert f32_bits(gpu_val) == f32_bits(np.float32(want)), (float(gpu_val), want)
