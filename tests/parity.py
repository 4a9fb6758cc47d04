"""Parity helpers: run the HIP path and the float64 oracle on the same inputs
and compare them to the bar the tests state.

Tolerances (written here once, used by every GPU parity test):
  * loss, z_loss (scalars and per-row "none" values): relative 1e-5; an
    oracle value of exactly 0 must be exactly 0 on the GPU; NaN and
    infinities must match.
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
import os

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
    inf_w = np.isinf(w)  # infinities must match exactly (value and sign)
    assert np.array_equal(g[inf_w], w[inf_w]) and not np.isinf(g[~inf_w]).any(), (
        f"{what}: infinities differ")
    m = ~nan_w & ~zero & ~inf_w
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
    nan_w = np.isnan(want)
    if nan_w.any() or np.isnan(g).any():
        bad_nan = np.isnan(g) != nan_w
        assert not bad_nan.any(), (
            f"{what}: NaN pattern differs at {int(bad_nan.sum())} elements, first at "
            f"{np.argwhere(bad_nan)[0].tolist()}")
        g = np.where(nan_w, 0.0, g)
        want = np.where(nan_w, 0.0, want)
        mag = np.where(nan_w, 0.0, mag)
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


def oracle_workers() -> int:
    """Threads for the oracle over row chunks: the host cores this process may
    use, at most 16 (numpy's array loops release the GIL)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_rows(x_host, t_host, *, weight=None, ignore_index=-100, label_smoothing=0.0,
                lse_square_scale=0.0, softcap=None, reduction="mean", want_grad=False,
                chunk=64, rows=None):
    """The oracle's per-row results (rows_forward) over every row of a batch
    (or the given rows), in row chunks spread over threads; the scales come
    from the whole batch's targets. Returns the merged RowResult fields and
    the target summary."""
    import concurrent.futures as cf
    V = x_host.shape[1]
    w = None if weight is None else np.asarray(weight, dtype=np.float64)
    t = np.asarray(t_host, dtype=np.int64)
    summ = summarize_targets(t, V, ignore_index, w, reduction)
    sel = np.arange(t.shape[0]) if rows is None else np.asarray(rows)
    n = sel.shape[0]
    out = dict(ce=np.zeros(n), zeta=np.zeros(n), argmax=np.zeros(n, dtype=np.int64),
               correct=np.zeros(n, dtype=bool))
    if want_grad:
        out["grad"] = np.zeros((n, V))
        out["mag"] = np.zeros((n, V))

    def one(a):
        b = min(n, a + chunk)
        r = rows_forward(x_host[sel[a:b]], t[sel[a:b]], V=V, alpha=summ.alpha, beta=summ.beta,
                         weight=w, ignore_index=ignore_index, label_smoothing=label_smoothing,
                         lse_square_scale=lse_square_scale, softcap=softcap,
                         want_grad=want_grad, want_mag=want_grad)
        out["ce"][a:b] = r.ce
        out["zeta"][a:b] = r.zeta
        out["argmax"][a:b] = r.argmax
        out["correct"][a:b] = r.correct
        if want_grad:
            out["grad"][a:b] = r.grad
            out["mag"][a:b] = r.mag

    with cf.ThreadPoolExecutor(oracle_workers()) as ex:
        list(ex.map(one, range(0, n, chunk)))
    return out, summ


class OracleRef:
    """Oracle results for a batch (optionally only for a sample of rows)."""

    def __init__(self, x_host, t_host, *, weight=None, ignore_index=-100, label_smoothing=0.0,
                 lse_square_scale=0.0, softcap=None, reduction="mean", rows=None,
                 want_grad=True, chunk=64):
        o, self.summ = oracle_rows(x_host, t_host, weight=weight, ignore_index=ignore_index,
                                   label_smoothing=label_smoothing,
                                   lse_square_scale=lse_square_scale, softcap=softcap,
                                   reduction=reduction, want_grad=want_grad, chunk=chunk,
                                   rows=rows)
        sel = np.arange(len(t_host)) if rows is None else np.asarray(rows)
        self.rows = sel
        self.not_counted = ~self.summ.counted[sel]
        self.ce, self.zeta = o["ce"], o["zeta"]
        self.argmax, self.correct = o["argmax"], o["correct"]
        self.grad = o.get("grad")
        self.mag = o.get("mag")
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
