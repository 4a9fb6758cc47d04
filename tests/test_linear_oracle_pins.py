"""Pins of the fused linear + cross-entropy oracle (CPU only).

The oracle (oracle/linear_oracle.py) composes a bias-free linear layer with
the cross-entropy oracle and takes the gradients by the chain rule. These
tests tie it to things other than itself:
  * torch CPU float64 autograd of F.cross_entropy(F.linear(hidden, weight))
    (the special case without softcap and z-loss, every reduction, class
    weights and label smoothing);
  * central finite differences of the oracle's own loss with every option
    on (softcap, z-loss, weights, smoothing), which checks the chain rule
    and the sign and transpose of both gradient products;
  * invariants: ignored rows have zero hidden gradient and do not depend
    on their hidden state; the logits equal hidden @ weight^T entry by entry.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import linear_forward

pytestmark = pytest.mark.filterwarnings("ignore")


def _inputs(rows, H, V, seed, n_ignored=0, scale=0.5):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, H)) * scale
    w = g.standard_normal((V, H)) * scale
    t = g.integers(0, V, rows).astype(np.int64)
    if n_ignored:
        t[g.choice(rows, n_ignored, replace=False)] = -100
    return x, w, t


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("use_weight", [False, True])
@pytest.mark.parametrize("eps", [0.0, 0.2])
def test_linear_matches_torch_cpu_float64(reduction, use_weight, eps):
    rows, H, V = 23, 9, 17
    x, w, t = _inputs(rows, H, V, 11, n_ignored=4)
    cw = np.random.default_rng(3).uniform(0.5, 2.0, V) if use_weight else None
    r = linear_forward(x, w, t, class_weight=cw, label_smoothing=eps, reduction=reduction)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    loss = F.cross_entropy(F.linear(xt, wt), torch.tensor(t),
                           weight=None if cw is None else torch.tensor(cw),
                           ignore_index=-100, label_smoothing=eps, reduction=reduction)
    loss.sum().backward()
    np.testing.assert_allclose(np.asarray(r.ce.loss), loss.detach().numpy(), rtol=1e-13,
                               atol=1e-13)
    np.testing.assert_allclose(r.grad_hidden, xt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r.grad_weight, wt.grad.numpy(), rtol=1e-12, atol=1e-14)


def _loss_scalar(x, w, t, **kw):
    r = linear_forward(x, w, t, want_grad=False, **kw)
    return float(np.sum(r.ce.loss))


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_linear_gradients_by_central_differences(reduction):
    rows, H, V = 6, 5, 7
    x, w, t = _inputs(rows, H, V, 5, n_ignored=1, scale=0.8)
    kw = dict(class_weight=np.linspace(0.5, 1.5, V), label_smoothing=0.1,
              lse_square_scale=1e-2, softcap=1.7, reduction=reduction)
    r = linear_forward(x, w, t, **kw)
    h = 1e-6
    for (i, j) in [(0, 0), (2, 3), (5, 4), (1, 1)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        fd = (_loss_scalar(xp, w, t, **kw) - _loss_scalar(xm, w, t, **kw)) / (2 * h)
        assert abs(fd - r.grad_hidden[i, j]) <= 1e-7 * max(1.0, abs(fd)), (i, j, fd)
    for (k, j) in [(0, 0), (3, 2), (6, 4), (t[0] if t[0] >= 0 else 2, 1)]:
        wp, wm = w.copy(), w.copy()
        wp[k, j] += h
        wm[k, j] -= h
        fd = (_loss_scalar(x, wp, t, **kw) - _loss_scalar(x, wm, t, **kw)) / (2 * h)
        assert abs(fd - r.grad_weight[k, j]) <= 1e-7 * max(1.0, abs(fd)), (k, j, fd)


def test_linear_ignored_rows():
    rows, H, V = 10, 4, 9
    x, w, t = _inputs(rows, H, V, 9)
    t[[1, 4, 7]] = -100
    r = linear_forward(x, w, t, label_smoothing=0.1, lse_square_scale=1e-3, softcap=3.0)
    assert np.all(r.grad_hidden[[1, 4, 7]] == 0.0)
    x2 = x.copy()
    x2[[1, 4, 7]] = 123.0                      # ignored rows' hidden states do not matter
    r2 = linear_forward(x2, w, t, label_smoothing=0.1, lse_square_scale=1e-3, softcap=3.0)
    assert r.ce.loss == r2.ce.loss
    np.testing.assert_array_equal(r.grad_weight, r2.grad_weight)


def test_linear_logits_entries():
    rows, H, V = 5, 6, 8
    x, w, t = _inputs(rows, H, V, 2)
    r = linear_forward(x, w, t)
    for i in range(rows):
        for k in range(V):
            assert r.logits[i, k] == pytest.approx(sum(x[i, j] * w[k, j] for j in range(H)),
                                                   rel=1e-14, abs=1e-14)
    assert np.all(r.logits_abs >= np.abs(r.logits) - 1e-12)


def test_linear_bf16_inputs_widen_exactly():
    rows, H, V = 4, 8, 6
    x, w, t = _inputs(rows, H, V, 4)
    xb = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
    wb = torch.tensor(w, dtype=torch.float32).to(torch.bfloat16)
    bits = lambda a: a.view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    r = linear_forward(bits(xb), bits(wb), t)
    r64 = linear_forward(xb.double().numpy(), wb.double().numpy(), t)
    assert r.ce.loss == r64.ce.loss
    np.testing.assert_array_equal(r.grad_hidden, r64.grad_hidden)


def test_tolerance_helpers_golden():
    """logits_abs = |hidden| @ |weight|^T and grad_magnitudes = (|G| @ |weight|,
    |G|^T @ |hidden|), which size every bar of the linear-path parity tests,
    against hand-computed values (tests/golden/tolerance_helpers.json): a
    transposed operand or a dropped absolute value fails here."""
    import json
    import os
    from oracle import grad_magnitudes, linear_forward
    path = os.path.join(os.path.dirname(__file__), "golden", "tolerance_helpers.json")
    c = json.load(open(path))["linear_case"]
    h = np.array(c["hidden"])
    w = np.array(c["weight"])
    G = np.array(c["G"])
    r = linear_forward(h, w, np.array([0, 2]), want_grad=False)
    np.testing.assert_array_equal(r.logits_abs, np.array(c["logits_abs"]))
    gh, gw = grad_magnitudes(h, w, G)
    np.testing.assert_array_equal(gh, np.array(c["grad_hidden_mag"]))
    np.testing.assert_array_equal(gw, np.array(c["grad_weight_mag"]))


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_row_chunked_form_equals_whole_batch(reduction):
    """linear_forward_rows (row blocks, global gradient scales, weight
    gradient summed block by block) gives linear_forward's values."""
    from oracle import grad_magnitudes, linear_forward_rows
    rng = np.random.default_rng(11)
    rows, H, V = 13, 6, 9
    x = rng.standard_normal((rows, H))
    w = rng.standard_normal((V, H))
    t = rng.integers(0, V, rows)
    t[[2, 7]] = -100
    cw = rng.uniform(0.5, 2.0, V)
    opts = dict(class_weight=cw, label_smoothing=0.1, lse_square_scale=0.01, softcap=4.0,
                reduction=reduction)
    full = linear_forward(x, w, t, **opts)
    sr = np.array([0, 2, 5, 12])
    sc = np.array([1, 8, 3])
    at = rng.integers(0, V, rows)
    part = linear_forward_rows(x, w, t, sample_rows=sr, sample_cols=sc, at_cols=at, row_chunk=4,
                               **opts)
    np.testing.assert_allclose(part.loss, full.ce.loss, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(part.z_loss, full.ce.z_loss, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(part.argmax, full.ce.argmax)
    assert part.n_correct == full.ce.n_correct and part.n_valid == full.ce.n_valid
    np.testing.assert_allclose(part.grad_hidden, full.grad_hidden[sr], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(part.grad_weight, full.grad_weight[sc], rtol=1e-12, atol=1e-15)
    srt = np.sort(full.logits, axis=1)
    np.testing.assert_allclose(part.top2, srt[:, ::-1][:, :2], rtol=1e-14)
    np.testing.assert_allclose(part.at_cols, full.logits[np.arange(rows), at], rtol=1e-14)
    np.testing.assert_allclose(part.logits_abs_max, full.logits_abs.max(axis=1), rtol=1e-14)
    mh, mw = grad_magnitudes(x, w, full.ce.grad)
    np.testing.assert_allclose(part.mag_hidden, mh[sr], rtol=1e-12)
    np.testing.assert_allclose(part.mag_weight, mw[sc], rtol=1e-12)
