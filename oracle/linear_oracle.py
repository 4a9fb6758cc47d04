"""Float64 CPU oracle for the linear layer fused with the cross-entropy.

TEST INFRASTRUCTURE. Like ce_oracle, this is a test reference, not the
product: only the test suite, the package entry's smoke check and the
benchmark's CPU-baseline leg may import it, and it shares nothing with the
HIP path.

What is computed
----------------
The Liger-Kernel page "Kernel Profile: CrossEntropy (Tier 3 -
Fused/Complex)", Classification, names the fused linear cross-entropy as the
kernel this one extends with a linear layer. Its plainest reading, taken
here: the logits are the output of a bias-free linear layer (the language
model head),

    logits = hidden @ weight^T          hidden (rows, H), weight (V, H),

and everything after is the cross-entropy of ce_oracle with the same
options (ignore_index, label smoothing, z-loss, softcap, class weights,
reductions). The gradients follow by the chain rule from G = d loss /
d logits (ce_oracle's gradient):

    d loss / d hidden = G @ weight,     d loss / d weight = G^T @ hidden.

Inputs are taken as stored (bfloat16 bit patterns or floats) and widened
exactly to float64; the products are float64 matrix products.

Error bounds for the tests (helpers below): a float32 evaluation of the
products differs from the float64 one by at most about K * 2^-24 times the
product of the absolute values (K the length of the sum), so the tests
size their tolerances from |hidden| @ |weight|^T and |G| @ |weight|,
|G|^T @ |hidden|, which this module also returns.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .ce_oracle import OracleResult, ce_forward, widen


@dataclass
class LinearResult:
    ce: OracleResult                  # the cross-entropy on the float64 logits
    logits: np.ndarray                # float64 (rows, V)
    grad_hidden: Optional[np.ndarray]  # float64 (rows, H)
    grad_weight: Optional[np.ndarray]  # float64 (V, H)
    logits_abs: np.ndarray            # |hidden| @ |weight|^T  (rows, V)


def linear_forward(hidden, weight, target, class_weight=None, ignore_index: int = -100,
                   label_smoothing: float = 0.0, lse_square_scale: float = 0.0,
                   softcap: Optional[float] = None, reduction: str = "mean",
                   want_grad: bool = True) -> LinearResult:
    """Loss, metrics and gradients of cross_entropy(hidden @ weight^T, target).

    hidden (rows, H) and weight (V, H) as stored (uint16 = bfloat16 bits,
    float32 or float64); class_weight (V,) or None.
    """
    x = widen(hidden)
    w = widen(weight)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("hidden must be (rows, H) and weight (V, H)")
    logits = x @ w.T
    res = ce_forward(logits, target, weight=class_weight, ignore_index=ignore_index,
                     label_smoothing=label_smoothing, lse_square_scale=lse_square_scale,
                     softcap=softcap, reduction=reduction, want_grad=want_grad)
    gh = gw = None
    if want_grad:
        G = res.grad
        gh = G @ w                      # chain rule through logits = hidden @ weight^T
        gw = G.T @ x
    return LinearResult(res, logits, gh, gw, np.abs(x) @ np.abs(w).T)


def grad_magnitudes(hidden, weight, G) -> tuple:
    """|G| @ |weight| and |G|^T @ |hidden|: the scale of the rounding error of
    the two gradient products (and of rounding G itself)."""
    x = np.abs(widen(hidden))
    w = np.abs(widen(weight))
    a = np.abs(np.asarray(G, dtype=np.float64))
    return a @ w, a.T @ x


@dataclass
class LinearRowsResult:
    """linear_forward evaluated in row chunks (every row's loss terms and
    argmax; gradients only for the sampled rows of hidden and classes of
    weight)."""
    loss: object                 # float64 scalar, or (rows,) for "none"
    z_loss: object
    token_accuracy: object
    argmax: np.ndarray           # int64 (rows,)
    n_valid: int
    n_correct: int
    D: float
    counted: np.ndarray          # bool (rows,)
    top2: np.ndarray             # float64 (rows, 2): the two largest logits of each row
    at_cols: Optional[np.ndarray]  # float64 (rows,): logits[i, at_cols[i]], or None
    logits_abs_max: np.ndarray   # float64 (rows,): max_k (|hidden| @ |weight|^T)_ik
    grad_hidden: np.ndarray      # float64 (len(sample_rows), H)
    grad_weight: np.ndarray      # float64 (len(sample_cols), H): rows sample_cols of d loss / d weight
    mag_hidden: np.ndarray       # |G| @ |weight| on sample_rows
    mag_weight: np.ndarray       # (|G|^T @ |hidden|) on sample_cols


def linear_forward_rows(hidden, weight, target, *, sample_rows, sample_cols, at_cols=None,
                        class_weight=None, ignore_index: int = -100,
                        label_smoothing: float = 0.0, lse_square_scale: float = 0.0,
                        softcap: Optional[float] = None, reduction: str = "mean",
                        row_chunk: int = 256) -> LinearRowsResult:
    """The definitions of linear_forward for batches whose (rows, V) float64
    logits do not fit at once: logits = hidden @ weight^T and the
    cross-entropy of each block of rows (ce_oracle.rows_forward, with the
    gradient scales of the whole batch from summarize_targets), then
    d loss / d hidden = G @ weight on sample_rows and
    d loss / d weight = G^T @ hidden on the classes sample_cols, the sum over
    rows taken block by block."""
    from .ce_oracle import reduce_rows, rows_forward, summarize_targets
    x = widen(hidden)
    w = widen(weight)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("hidden must be (rows, H) and weight (V, H)")
    rows, H = x.shape
    V = w.shape[0]
    t = np.asarray(target, dtype=np.int64)
    summ = summarize_targets(t, V, ignore_index, class_weight, reduction)
    sample_rows = np.asarray(sample_rows, dtype=np.int64)
    sample_cols = np.asarray(sample_cols, dtype=np.int64)
    ce = np.zeros(rows)
    zeta = np.zeros(rows)
    argmax = np.full(rows, -1, dtype=np.int64)
    correct = np.zeros(rows, dtype=bool)
    top2 = np.zeros((rows, 2))
    at = None if at_cols is None else np.zeros(rows)
    absmax = np.zeros(rows)
    gh = np.zeros((sample_rows.size, H))
    mh = np.zeros((sample_rows.size, H))
    gw = np.zeros((sample_cols.size, H))
    mw = np.zeros((sample_cols.size, H))
    xa, wa = np.abs(x), np.abs(w)
    for r0 in range(0, rows, row_chunk):
        r1 = min(rows, r0 + row_chunk)
        z = x[r0:r1] @ w.T
        rr = rows_forward(z, t[r0:r1], V=V, alpha=summ.alpha, beta=summ.beta,
                          weight=class_weight, ignore_index=ignore_index,
                          label_smoothing=label_smoothing, lse_square_scale=lse_square_scale,
                          softcap=softcap, want_grad=True)
        ce[r0:r1], zeta[r0:r1] = rr.ce, rr.zeta
        argmax[r0:r1], correct[r0:r1] = rr.argmax, rr.correct
        srt = np.sort(z, axis=1)
        top2[r0:r1, 0] = srt[:, -1]
        top2[r0:r1, 1] = srt[:, -2] if V > 1 else -np.inf
        if at is not None:
            c = np.asarray(at_cols[r0:r1], dtype=np.int64)
            ok = (c >= 0) & (c < V)
            at[r0:r1] = np.where(ok, z[np.arange(r1 - r0), np.clip(c, 0, V - 1)], np.nan)
        absmax[r0:r1] = (xa[r0:r1] @ wa.T).max(axis=1)
        G = rr.grad
        sel = np.nonzero((sample_rows >= r0) & (sample_rows < r1))[0]
        if sel.size:
            Gs = G[sample_rows[sel] - r0]
            gh[sel] = Gs @ w
            mh[sel] = np.abs(Gs) @ wa
        Gc = G[:, sample_cols]
        gw += Gc.T @ x[r0:r1]
        mw += np.abs(Gc).T @ xa[r0:r1]
    loss, z_loss, acc, n_correct = reduce_rows(ce, zeta, correct, summ.counted, summ.n, summ.D,
                                               reduction)
    return LinearRowsResult(loss, z_loss, acc, argmax, summ.n, n_correct, summ.D, summ.counted,
                            top2, at, absmax, gh, gw, mh, mw)
