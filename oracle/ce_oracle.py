"""Float64 CPU oracle for fused softmax cross-entropy forward + gradient.

TEST INFRASTRUCTURE. This module is the reference the kernels are tested
against, not the product: only the test suite, the package entry's smoke
check and the benchmark's CPU-baseline leg may import it. The product path (HIP kernels behind the C ABI) never
calls it, and the two share no code, tables or helpers.

What is computed, and where the pages define it
-----------------------------------------------
Sources: the Liger-Kernel page "Kernel Profile: CrossEntropy (Tier 3 -
Fused/Complex)" (called the Liger CE profile below) and the tt-mlir pull
request page "[tt-crank] fuse cross entropy onto the ttml
cross_entropy_fw/bw composites" (#9324, called the PR #9324 page below),
which also quotes the description of the aten fallback lowerings of
PR #9339.

* Inputs and options -- Liger CE profile, Forward Pass (forward_inputs) and
  Module Parameters: logits of shape (rows, V), integer targets of shape
  (rows,), optional class weights (V,), ignore_index (default -100),
  label_smoothing, lse_square_scale (z-loss), reduction in
  {"mean", "sum", "none"}, softcap (None = off).
* Outputs -- Liger CE profile, Forward Pass (forward_outputs): loss (scalar,
  or per row for "none"), z_loss, token_accuracy, predicted tokens (argmax).
* Max-shifted log-sum-exp -- PR #9324 page, quoted #9339 description: the
  log-softmax must be computed as x - (m + log sum exp(x - m)), never as
  log(softmax(x)).
* Loss components -- Liger CE profile, Key Patterns ("Multiple loss
  components"): cross entropy, label smoothing and z-loss each add to the
  loss and to the gradient.
* Gradient -- Liger CE profile, Backward Pass and Key Patterns
  ("Gradient-in-forward trick"): the forward produces d loss / d logits; the
  backward only multiplies it by grad_output.
* All-ignored mean -- PR #9324 page, Copilot suppressed comments on
  _compile.py (mean reduction with total_weight zero) and the quoted #9339
  description (row count clamped so an all-ignored batch gives zero
  gradients): the mean loss stays NaN, the gradients are exactly zero.

Readings where the pages are silent (each is a plain reading):

* Formula: the PyTorch cross-entropy convention, which the PR #9324 page
  uses as ground truth (tests "against CPU") and the Liger CE profile
  benchmarks against ("huggingface" provider).  With z = softcapped logits,
  p = softmax(z), log p = z - lse, eps = label_smoothing, w = class weights
  (all ones when absent), W = sum_k w_k:
      l_i = -(1 - eps) * w_y * log p_y - (eps / V) * sum_k w_k * log p_k
  and the mean divides sum_i l_i by D = sum over counted rows of w_y.
  With eps = 0 (the Module Parameters default: no smoothing) the second
  term is absent, not 0 times the sum: a -inf logit elsewhere in the row
  leaves the loss finite, as torch's cross_entropy does.
* z-loss: zeta_i = lse_square_scale * lse_i**2, not class-weighted, over the
  softcapped logits; the mean divides sum_i zeta_i by n (counted rows).
  The returned loss includes it; z_loss returns it alone.
* Softcap: z = c * tanh(x / c) for c > 0, applied first; the gradient
  chains through it with the factor 1 - tanh(x / c)**2.
* argmax: over the raw stored logits, lowest index on ties; -1 on rows that
  are not counted. A NaN ranks above every number (the ordering of
  numpy.argmax and torch.argmax), so a counted row holding a NaN has the
  index of its first NaN as argmax; its loss and gradient are NaN (every
  exponential of the row is).
* Non-finite logits in counted rows are taken as IEEE arithmetic gives
  them: a +inf logit makes the max shift inf and the row's loss and
  gradient NaN, a -inf logit has probability 0.
* token_accuracy: n_correct / n for "mean" and "sum" (NaN when n = 0); the
  per-row 0/1 value for "none".
* Rows whose target equals ignore_index are never read (they may hold
  non-finite values) and get zero loss, zero z-loss and zero gradient.
* Rows whose target is neither ignore_index nor in [0, V) are "bad": not
  counted in n, D or n_correct, zero gradient, argmax -1, and NaN loss and
  z-loss so that any reduction over them is NaN.
* Gradient scales: alpha = 1 / D and beta = 1 / n for "mean", with
  alpha := 0 when D == 0 and beta := 0 when n == 0 (zero gradients, NaN
  loss); alpha = beta = 1 for "sum" and "none".
* Output rounding is not modelled: every result is float64 (the unrounded
  value), integers are int64.

The computation is the plain definition, row by row in float64, with no
online rescaling and no chunk combining: a reader can check each line
against the formulas above.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

REDUCTIONS = ("mean", "sum", "none")


def widen(x) -> np.ndarray:
    """Widen stored logits exactly to float64.

    A uint16 array is taken as raw bfloat16 bit patterns (the upper half of
    an IEEE binary32), which widen exactly; float32/float64 widen exactly.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype not in (np.float32, np.float64):
        raise TypeError(f"unsupported logits dtype {x.dtype}")
    return x.astype(np.float64)


@dataclass
class TargetSummary:
    """Counted rows and the mean denominators, from the targets alone."""
    counted: np.ndarray      # bool (rows,): target != ignore_index and 0 <= target < V
    bad: np.ndarray          # bool (rows,): target != ignore_index and out of [0, V)
    n: int                   # number of counted rows
    D: float                 # sum over counted rows of w[target] (== n without weights)
    alpha: float             # gradient scale of the cross-entropy part
    beta: float              # gradient scale of the z-loss part


def summarize_targets(target, V: int, ignore_index: int = -100, weight=None,
                      reduction: str = "mean") -> TargetSummary:
    """Counted rows, n, D and the gradient scales alpha, beta.

    PR #9324 page (Copilot comments on the mean reduction): the mean divides
    by total_weight; when it is zero the gradient must stay zero.
    """
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {REDUCTIONS}")
    t = np.asarray(target, dtype=np.int64)
    not_ignored = t != ignore_index
    in_range = (t >= 0) & (t < V)
    counted = not_ignored & in_range
    bad = not_ignored & ~in_range
    n = int(np.count_nonzero(counted))
    if weight is None:
        D = float(n)
    else:
        w = np.asarray(weight, dtype=np.float64)
        D = float(np.sum(w[t[counted]]))
    if reduction == "mean":
        alpha = 1.0 / D if D != 0.0 else 0.0
        beta = 1.0 / n if n != 0 else 0.0
    else:
        alpha = 1.0
        beta = 1.0
    return TargetSummary(counted, bad, n, D, alpha, beta)


@dataclass
class RowResult:
    """Per-row quantities for a block of rows."""
    ce: np.ndarray        # float64 (r,): l_i (0 on ignored rows, NaN on bad rows)
    zeta: np.ndarray      # float64 (r,): lse_square_scale * lse_i**2 (same conventions)
    lse: np.ndarray       # float64 (r,): log-sum-exp over softcapped logits (NaN if not counted)
    argmax: np.ndarray    # int64 (r,): first index of the raw maximum, -1 if not counted
    correct: np.ndarray   # bool (r,): argmax == target on counted rows
    grad: Optional[np.ndarray]  # float64 (r, V) d(loss)/d(logits), or None
    mag: Optional[np.ndarray] = None  # float64 (r, V) sum of |gradient terms| (want_mag)


def rows_forward(x_rows, target_rows, *, V: int, alpha: float, beta: float,
                 weight=None, ignore_index: int = -100, label_smoothing: float = 0.0,
                 lse_square_scale: float = 0.0, softcap: Optional[float] = None,
                 want_grad: bool = True, want_mag: bool = False) -> RowResult:
    """Loss terms, argmax and gradient of a block of rows.

    alpha and beta come from summarize_targets over the whole batch, so a
    sample of rows gives the same values as the full computation.

    want_mag also returns, per element, the sum of the absolute values of
    the gradient's terms (alpha (1-eps) w_y p_k, alpha (1-eps) w_y [k = y],
    alpha (eps/V) W p_k, alpha (eps/V) w_k, beta 2 lam |lse| p_k) times the
    softcap factor: the scale at which cancellation between them loses
    precision in a float32 evaluation. It is used only to size the bfloat16
    gradient tolerance.
    """
    x = widen(x_rows)
    if x.ndim != 2 or x.shape[1] != V:
        raise ValueError("x_rows must have shape (r, V)")
    t = np.asarray(target_rows, dtype=np.int64)
    r = x.shape[0]
    eps = float(label_smoothing)
    lam = float(lse_square_scale)
    c = float(softcap) if softcap else 0.0
    w = np.ones(V) if weight is None else np.asarray(weight, dtype=np.float64)
    W = float(np.sum(w))

    not_ignored = t != ignore_index
    in_range = (t >= 0) & (t < V)
    counted = not_ignored & in_range
    bad = not_ignored & ~in_range

    ce = np.zeros(r)
    zeta = np.zeros(r)
    lse_out = np.full(r, np.nan)
    argmax = np.full(r, -1, dtype=np.int64)
    correct = np.zeros(r, dtype=bool)
    grad = np.zeros((r, V)) if want_grad else None
    mag = np.zeros((r, V)) if want_mag else None
    ce[bad] = np.nan
    zeta[bad] = np.nan

    idx = np.nonzero(counted)[0]
    if idx.size:
        xv = x[idx]                      # ignored and bad rows are never read
        y = t[idx]
        if c > 0.0:
            th = np.tanh(xv / c)
            z = c * th                   # softcap first
        else:
            z = xv
        m = np.max(z, axis=1, keepdims=True)                  # max shift
        s = np.sum(np.exp(z - m), axis=1, keepdims=True)
        lse = m + np.log(s)
        logp = z - lse                                        # log-softmax
        logp_y = logp[np.arange(idx.size), y]
        w_y = w[y]
        ce_rows = -(1.0 - eps) * w_y * logp_y
        if eps > 0.0:                                         # smoothing term only when on
            ce_rows = ce_rows - (eps / V) * (logp @ w)
        zeta_rows = lam * lse[:, 0] ** 2
        ce[idx] = ce_rows
        zeta[idx] = zeta_rows
        lse_out[idx] = lse[:, 0]
        am = np.argmax(xv, axis=1)                            # raw logits, first maximum
        argmax[idx] = am
        correct[idx] = am == y
        if want_grad:
            p = np.exp(logp)
            onehot = np.zeros_like(p)
            onehot[np.arange(idx.size), y] = 1.0
            g_ce = (1.0 - eps) * w_y[:, None] * (p - onehot) + (eps / V) * (W * p - w[None, :])
            g_z = 2.0 * lam * lse * p
            g = alpha * g_ce + beta * g_z
            if c > 0.0:
                g = g * (1.0 - th * th)                       # chain through z = c tanh(x/c)
            grad[idx] = g
        if want_mag:
            p = np.exp(logp)
            onehot = np.zeros_like(p)
            onehot[np.arange(idx.size), y] = 1.0
            mg = (abs(alpha) * (1.0 - eps) * w_y[:, None] * (p + onehot)
                  + abs(alpha) * (eps / V) * (W * p + w[None, :])
                  + abs(beta) * 2.0 * lam * np.abs(lse) * p)
            if c > 0.0:
                mg = mg * (1.0 - th * th)
            mag[idx] = mg
    return RowResult(ce, zeta, lse_out, argmax, correct, grad, mag)


@dataclass
class OracleResult:
    loss: object            # float64 scalar, or (rows,) for "none"
    z_loss: object          # same shape as loss
    token_accuracy: object  # float64 scalar, or (rows,) for "none"
    argmax: np.ndarray      # int64 (rows,)
    n_valid: int
    n_correct: int
    D: float
    alpha: float
    beta: float
    ce: np.ndarray          # per-row l_i
    zeta: np.ndarray        # per-row zeta_i
    grad: Optional[np.ndarray]
    bad: np.ndarray


def reduce_rows(ce: np.ndarray, zeta: np.ndarray, correct: np.ndarray, counted: np.ndarray,
                n: int, D: float, reduction: str):
    """Reductions of the per-row terms (Liger CE profile, forward_outputs;
    PR #9324 page, fallback lowering: none returns rows, sum/mean reduce).

    Divisions follow IEEE float64: 0/0 is NaN, which is the all-ignored mean.
    """
    with np.errstate(divide="ignore", invalid="ignore"):
        n_correct = int(np.count_nonzero(correct & counted))
        if reduction == "none":
            loss = ce + zeta
            z_loss = zeta.copy()
            acc = (correct & counted).astype(np.float64)
            return loss, z_loss, acc, n_correct
        sce = float(np.sum(ce))
        sz = float(np.sum(zeta))
        acc = np.float64(n_correct) / np.float64(n)
        if reduction == "sum":
            return sce + sz, sz, acc, n_correct
        loss = np.float64(sce) / np.float64(D) + np.float64(sz) / np.float64(n)
        z_loss = np.float64(sz) / np.float64(n)
        return float(loss), float(z_loss), acc, n_correct


def ce_forward(logits, target, weight=None, ignore_index: int = -100,
               label_smoothing: float = 0.0, lse_square_scale: float = 0.0,
               softcap: Optional[float] = None, reduction: str = "mean",
               want_grad: bool = True, row_chunk: int = 256) -> OracleResult:
    """Whole-batch forward: losses, metrics and d(loss)/d(logits).

    The gradient is that of the returned loss (cross entropy plus z-loss)
    with grad_output = 1 (Liger CE profile, Backward Pass: the forward
    stores the gradient; the backward only rescales it).
    """
    x = np.asarray(logits)
    if x.ndim != 2:
        raise ValueError("logits must be 2-D (rows, V)")
    rows, V = x.shape
    if not (0.0 <= label_smoothing <= 1.0):
        raise ValueError("label_smoothing must be in [0, 1]")
    t = np.asarray(target, dtype=np.int64)
    summ = summarize_targets(t, V, ignore_index, weight, reduction)
    ce = np.zeros(rows)
    zeta = np.zeros(rows)
    argmax = np.full(rows, -1, dtype=np.int64)
    correct = np.zeros(rows, dtype=bool)
    grad = np.zeros((rows, V)) if want_grad else None
    for r0 in range(0, rows, row_chunk):
        r1 = min(rows, r0 + row_chunk)
        rr = rows_forward(x[r0:r1], t[r0:r1], V=V, alpha=summ.alpha, beta=summ.beta,
                          weight=weight, ignore_index=ignore_index,
                          label_smoothing=label_smoothing, lse_square_scale=lse_square_scale,
                          softcap=softcap, want_grad=want_grad)
        ce[r0:r1] = rr.ce
        zeta[r0:r1] = rr.zeta
        argmax[r0:r1] = rr.argmax
        correct[r0:r1] = rr.correct
        if want_grad:
            grad[r0:r1] = rr.grad
    loss, z_loss, acc, n_correct = reduce_rows(ce, zeta, correct, summ.counted, summ.n,
                                               summ.D, reduction)
    return OracleResult(loss, z_loss, acc, argmax, summ.n, n_correct, summ.D, summ.alpha,
                        summ.beta, ce, zeta, grad, summ.bad)


def ce_backward(grad, grad_output, per_row: bool = False) -> np.ndarray:
    """Backward: the stored gradient times grad_output (a scalar, or one value
    per row for reduction "none").  Liger CE profile, Backward Pass."""
    g = np.asarray(grad, dtype=np.float64)
    go = np.asarray(grad_output, dtype=np.float64)
    if per_row:
        return g * go.reshape(-1, 1)
    return g * go.reshape(())
