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
