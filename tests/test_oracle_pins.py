"""Pins for the float64 oracle: each check ties it to something other than
itself (closed forms, brute force at 50 digits, finite differences, a
library routine in a special case, exact invariants), so that a dropped
term, a wrong sign or a wrong index in the oracle fails at least one.

All of these run on the CPU.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

from oracle import ce_backward, ce_forward, rows_forward, summarize_targets, widen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _eval(expr):
    ns = {"log": math.log, "tanh": math.tanh, "atanh": math.atanh, "nan": math.nan}
    return float(eval(expr, {"__builtins__": {}}, ns))  # closed-form fixture strings only


# ---------------------------------------------------------------------------
# Worked examples with hand-derived closed forms (tests/golden)
# ---------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    x = np.array([[_eval(e) for e in case["x_expr"]]])
    t = np.array([case["target"]])
    w = np.array(case["weight"]) if "weight" in case else None
    r = ce_forward(x, t, weight=w, label_smoothing=case.get("label_smoothing", 0.0),
                   lse_square_scale=case.get("lse_square_scale", 0.0),
                   softcap=case.get("softcap"), reduction=case["reduction"])
    want = _eval(case["loss"])
    if math.isnan(want):
        assert math.isnan(r.loss)
    else:
        assert r.loss == pytest.approx(want, rel=1e-13, abs=1e-14)
    if "z_loss" in case:
        assert r.z_loss == pytest.approx(_eval(case["z_loss"]), rel=1e-13)
    g = np.array([_eval(e) for e in case["grad"]])
    np.testing.assert_allclose(r.grad[0], g, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Special case that reduces to a library routine: torch CPU float64
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("use_weight", [False, True])
@pytest.mark.parametrize("eps", [0.0, 0.1, 1.0])
def test_matches_torch_cpu_float64(reduction, use_weight, eps):
    rng = _rng(7)
    rows, V = 37, 53
    x = rng.standard_normal((rows, V)) * 2.0
    t = rng.integers(0, V, rows)
    t[rng.choice(rows, 5, replace=False)] = -100
    w = rng.uniform(0.5, 2.0, V) if use_weight else None
    r = ce_forward(x, t, weight=w, label_smoothing=eps, reduction=reduction)

    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64) if use_weight else None
    ref = torch.nn.functional.cross_entropy(xt, torch.tensor(t), weight=wt, ignore_index=-100,
                                            reduction=reduction, label_smoothing=eps)
    if reduction == "none":
        np.testing.assert_allclose(r.loss, ref.detach().numpy(), rtol=1e-12, atol=1e-13)
        ref.sum().backward()
    else:
        assert r.loss == pytest.approx(ref.item(), rel=1e-12)
        ref.backward()
    np.testing.assert_allclose(r.grad, xt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_all_ignored_matches_torch():
    x = _rng(3).standard_normal((6, 9))
    t = np.full(6, -100)
    r = ce_forward(x, t, reduction="mean")
    xt = torch.tensor(x, requires_grad=True)
    ref = torch.nn.functional.cross_entropy(xt, torch.tensor(t), reduction="mean")
    ref.backward()
    assert math.isnan(r.loss) and math.isnan(ref.item())
    assert np.all(r.grad == 0.0) and np.all(xt.grad.numpy() == 0.0)


def test_argmax_matches_torch_first_occurrence():
    rng = _rng(11)
    x = rng.integers(-3, 3, (64, 40)).astype(np.float64)  # many ties
    t = rng.integers(0, 40, 64)
    r = ce_forward(x, t, reduction="none")
    np.testing.assert_array_equal(r.argmax, torch.argmax(torch.tensor(x), dim=1).numpy())


# ---------------------------------------------------------------------------
# Brute force at 50 digits on the definitions (V <= 16), gradient by
# central differences: independent of the oracle's analytic gradient.
# ---------------------------------------------------------------------------

def _mp_row_loss(xrow, y, V, w, eps, lam, c):
    mpmath.mp.dps = 50
    z = [c * mpmath.tanh(xi / c) if c else xi for xi in xrow]
    lse = mpmath.log(mpmath.fsum(mpmath.e ** zi for zi in z))
    logp = [zi - lse for zi in z]
    ce = -(1 - eps) * w[y] * logp[y] - mpmath.mpf(eps) / V * mpmath.fsum(w[k] * logp[k] for k in range(V))
    return ce, lam * lse ** 2


def _mp_batch_loss(X, T, V, w, eps, lam, c, reduction):
    tot_ce, tot_z, D, n = 0, 0, 0, 0
    for row, y in zip(X, T):
        if y == -100:
            continue
        ce, zt = _mp_row_loss(row, int(y), V, w, eps, lam, c)
        tot_ce += ce
        tot_z += zt
        D += w[int(y)]
        n += 1
    if reduction == "sum":
        return tot_ce + tot_z
    return tot_ce / D + tot_z / n


@pytest.mark.parametrize("cfg", [
    dict(V=5, eps=0.0, lam=0.0, c=0.0, weighted=False, reduction="sum"),
    dict(V=7, eps=0.15, lam=0.0, c=0.0, weighted=True, reduction="mean"),
    dict(V=11, eps=0.0, lam=0.01, c=0.0, weighted=False, reduction="mean"),
    dict(V=16, eps=0.3, lam=0.02, c=3.0, weighted=True, reduction="mean"),
    dict(V=9, eps=0.1, lam=0.05, c=1.5, weighted=True, reduction="sum"),
])
def test_bruteforce_mpmath(cfg):
    V = cfg["V"]
    rng = _rng(100 + V)
    rows = 3
    X = rng.standard_normal((rows, V)) * 2.0
    T = rng.integers(0, V, rows)
    T[1] = -100
    w = rng.uniform(0.5, 2.0, V) if cfg["weighted"] else np.ones(V)
    r = ce_forward(X, T, weight=w if cfg["weighted"] else None, label_smoothing=cfg["eps"],
                   lse_square_scale=cfg["lam"], softcap=cfg["c"] or None, reduction=cfg["reduction"])
    mpmath.mp.dps = 50
    Xm = [[mpmath.mpf(float(v)) for v in row] for row in X]
    wm = [mpmath.mpf(float(v)) for v in w]
    args = (T, V, wm, mpmath.mpf(cfg["eps"]), mpmath.mpf(cfg["lam"]), mpmath.mpf(cfg["c"]),
            cfg["reduction"])
    L = _mp_batch_loss(Xm, *args)
    assert r.loss == pytest.approx(float(L), rel=1e-13)
    # per-row none values from the same definition
    rn = ce_forward(X, T, weight=w if cfg["weighted"] else None, label_smoothing=cfg["eps"],
                    lse_square_scale=cfg["lam"], softcap=cfg["c"] or None, reduction="none")
    for i in range(rows):
        if T[i] == -100:
            assert rn.loss[i] == 0.0
            continue
        ce, zt = _mp_row_loss(Xm[i], int(T[i]), V, *args[2:6])
        assert rn.loss[i] == pytest.approx(float(ce + zt), rel=1e-13)
        assert rn.z_loss[i] == pytest.approx(float(zt), rel=1e-13, abs=1e-300)
    # gradient: central differences of the 50-digit loss
    h = mpmath.mpf("1e-20")
    for i in range(rows):
        for k in range(V):
            Xp = [row[:] for row in Xm]
            Xn = [row[:] for row in Xm]
            Xp[i][k] += h
            Xn[i][k] -= h
            d = (_mp_batch_loss(Xp, *args) - _mp_batch_loss(Xn, *args)) / (2 * h)
            assert r.grad[i, k] == pytest.approx(float(d), rel=1e-10, abs=1e-15)


def test_argmax_exhaustive_ties():
    # every pattern of a 4-wide row over a 3-value alphabet: the first maximum wins
    vals = [-1.0, 0.0, 2.0]
    rows = []
    for a in vals:
        for b in vals:
            for c in vals:
                for d in vals:
                    rows.append([a, b, c, d])
    X = np.array(rows)
    r = ce_forward(X, np.zeros(len(rows), dtype=np.int64), reduction="none")
    for row, am in zip(rows, r.argmax):
        mx = max(row)
        assert am == row.index(mx)


# ---------------------------------------------------------------------------
# Closed forms and invariants at sizes beyond brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("lam", [0.0, 1e-3])
def test_uniform_logits(eps, lam):
    rows, V, a = 4, 1000, 1.7
    x = np.full((rows, V), a)
    t = np.array([0, 999, 500, 3])
    r = ce_forward(x, t, label_smoothing=eps, lse_square_scale=lam, reduction="none")
    np.testing.assert_allclose(r.ce, np.log(V), rtol=1e-13)
    np.testing.assert_allclose(r.zeta, lam * (a + np.log(V)) ** 2, rtol=1e-13)
    want = (1 - eps) * (1.0 / V - np.eye(V)[t]) + 2 * lam * (a + np.log(V)) / V
    np.testing.assert_allclose(r.grad, want, rtol=1e-11, atol=1e-15)


def test_uniform_logits_weighted():
    V = 64
    w = _rng(5).uniform(0.5, 2.0, V)
    x = np.zeros((2, V))
    t = np.array([3, 40])
    eps = 0.25
    r = ce_forward(x, t, weight=w, label_smoothing=eps, reduction="none")
    want = np.log(V) * ((1 - eps) * w[t] + eps * w.sum() / V)
    np.testing.assert_allclose(r.ce, want, rtol=1e-13)


@pytest.mark.parametrize("weighted", [False, True])
def test_gradient_row_sums(weighted):
    rng = _rng(21)
    rows, V = 8, 300
    x = rng.standard_normal((rows, V)) * 3
    t = rng.integers(0, V, rows)
    w = rng.uniform(0.5, 2.0, V) if weighted else None
    lam, c = 1e-2, 4.0
    r = ce_forward(x, t, weight=w, label_smoothing=0.2, lse_square_scale=lam, softcap=c,
                   reduction="mean")
    chain = 1 - np.tanh(x / c) ** 2
    s = (r.grad / chain).sum(axis=1)
    summ = summarize_targets(t, V, weight=w, reduction="mean")
    rr = rows_forward(x, t, V=V, alpha=1, beta=1, weight=w, label_smoothing=0.2,
                      lse_square_scale=lam, softcap=c, want_grad=False)
    np.testing.assert_allclose(s, summ.beta * 2 * lam * rr.lse, rtol=1e-9, atol=1e-13)


def test_smoothed_target_identity():
    rng = _rng(31)
    rows, V, eps = 5, 77, 0.3
    x = rng.standard_normal((rows, V))
    t = rng.integers(0, V, rows)
    r = ce_forward(x, t, label_smoothing=eps, reduction="none")
    logp = x - np.log(np.exp(x).sum(axis=1, keepdims=True))
    q = (1 - eps) * np.eye(V)[t] + eps / V
    np.testing.assert_allclose(r.ce, -(q * logp).sum(axis=1), rtol=1e-12)
    np.testing.assert_allclose(r.grad, np.exp(logp) - q, atol=1e-14)


def test_shift_invariance():
    rng = _rng(41)
    x = rng.standard_normal((6, 50))
    t = rng.integers(0, 50, 6)
    w = rng.uniform(0.5, 2, 50)
    a = ce_forward(x, t, weight=w, label_smoothing=0.1, reduction="none")
    b = ce_forward(x + 37.5, t, weight=w, label_smoothing=0.1, reduction="none")
    np.testing.assert_allclose(a.ce, b.ce, rtol=1e-12)
    np.testing.assert_allclose(a.grad, b.grad, atol=1e-14)


def test_softcap_is_applied_first_and_limits():
    rng = _rng(51)
    x = rng.standard_normal((4, 40)) * 5
    t = rng.integers(0, 40, 4)
    c = 7.0
    a = ce_forward(x, t, softcap=c, lse_square_scale=1e-3, label_smoothing=0.1, reduction="none")
    b = ce_forward(c * np.tanh(x / c), t, lse_square_scale=1e-3, label_smoothing=0.1, reduction="none")
    np.testing.assert_allclose(a.loss, b.loss, rtol=1e-13)
    np.testing.assert_allclose(a.grad, b.grad * (1 - np.tanh(x / c) ** 2), atol=1e-15)
    big = ce_forward(x, t, softcap=1e7, reduction="none")
    off = ce_forward(x, t, reduction="none")
    np.testing.assert_allclose(big.loss, off.loss, rtol=1e-9)
    np.testing.assert_allclose(big.grad, off.grad, atol=1e-9)


def test_ignored_rows_never_read_and_zero():
    rng = _rng(61)
    x = rng.standard_normal((8, 30))
    t = rng.integers(0, 30, 8)
    t[[1, 4, 6]] = -100
    x[1] = np.nan
    x[4] = np.inf
    x[6, 3] = -np.inf
    for red in ("mean", "sum", "none"):
        r = ce_forward(x, t, reduction=red, lse_square_scale=1e-2)
        assert np.all(np.isfinite(r.loss))
        assert np.all(r.grad[[1, 4, 6]] == 0.0)
        assert np.all(np.isfinite(r.grad))
        assert list(r.argmax[[1, 4, 6]]) == [-1, -1, -1]
    r = ce_forward(x, t, reduction="mean")
    assert r.n_valid == 5


def test_all_ignored_with_nonfinite_logits():
    x = np.full((512, 16), np.nan)
    x[1::4] = np.inf
    x[2::4] = -np.inf
    t = np.full(512, -100)
    r = ce_forward(x, t, reduction="mean", lse_square_scale=1e-4)
    assert math.isnan(r.loss) and math.isnan(r.z_loss) and math.isnan(r.token_accuracy)
    assert np.all(r.grad == 0.0) and not np.signbit(r.grad).any()
    assert r.n_valid == 0 and r.n_correct == 0
    s = ce_forward(x, t, reduction="sum")
    assert s.loss == 0.0 and math.isnan(s.token_accuracy)


def test_large_logit_spike_rows():
    rng = _rng(71)
    V = 4096
    x = rng.standard_normal((2, V))
    t = np.array([10, 20])
    x[0, 10] = 80.0   # spike at the target
    x[1, 99] = 80.0   # spike elsewhere
    r = ce_forward(x, t, reduction="none")
    xo = np.delete(x[0], 10)
    assert r.ce[0] == pytest.approx(np.log1p(np.exp(xo - 80.0).sum()), abs=1e-15)
    assert r.ce[1] == pytest.approx(80.0 - x[1, 20] + np.log1p(np.exp(np.delete(x[1], 99) - 80).sum()),
                                    rel=1e-14)
    assert abs(r.grad[0, 10]) < 1e-20
    assert r.grad[1, 99] == pytest.approx(1.0, abs=1e-20)
    assert np.all(np.isfinite(r.grad))


def test_full_smoothing_ignores_target():
    rng = _rng(81)
    x = rng.standard_normal((3, 25))
    a = ce_forward(x, np.array([0, 1, 2]), label_smoothing=1.0, reduction="none")
    b = ce_forward(x, np.array([24, 7, 13]), label_smoothing=1.0, reduction="none")
    np.testing.assert_allclose(a.loss, b.loss, rtol=1e-14)
    np.testing.assert_allclose(a.grad, b.grad, atol=1e-16)


def test_counts_and_accuracy():
    rng = _rng(91)
    rows, V = 200, 10
    x = rng.standard_normal((rows, V))
    t = rng.integers(0, V, rows)
    ign = rng.choice(rows, 20, replace=False)
    t[ign] = -100
    t[:30] = np.argmax(x[:30], axis=1)
    t[ign] = -100
    r = ce_forward(x, t, reduction="mean")
    assert r.n_valid == rows - 20
    am = np.argmax(x, axis=1)
    nc = int(np.sum((am == t) & (t != -100)))
    assert r.n_correct == nc
    assert r.token_accuracy == nc / (rows - 20)


def test_bad_targets():
    x = _rng(93).standard_normal((4, 6))
    t = np.array([0, 6, -1, -100])
    r = ce_forward(x, t, reduction="none")
    assert r.bad.tolist() == [False, True, True, False]
    assert math.isnan(r.loss[1]) and math.isnan(r.loss[2]) and r.loss[3] == 0.0
    assert np.all(r.grad[1:] == 0.0)
    assert list(r.argmax) == [int(np.argmax(x[0])), -1, -1, -1]
    m = ce_forward(x, t, reduction="mean")
    assert math.isnan(m.loss) and m.n_valid == 1


def test_mean_scale_and_zero_weight_guard():
    x = _rng(95).standard_normal((3, 5))
    t = np.array([1, 2, 3])
    w = np.array([1.0, 0.0, 0.0, 0.0, 1.0])
    r = ce_forward(x, t, weight=w, reduction="mean")   # D == 0 with n == 3
    assert r.D == 0.0 and r.alpha == 0.0
    assert np.all(r.grad == 0.0)


def test_backward_scales():
    x = _rng(97).standard_normal((5, 12))
    t = np.arange(5)
    r = ce_forward(x, t, reduction="none")
    go = np.array([1.0, 2.0, 0.0, -0.5, 3.0])
    np.testing.assert_array_equal(ce_backward(r.grad, go, per_row=True), r.grad * go[:, None])
    np.testing.assert_array_equal(ce_backward(r.grad, 0.37), r.grad * 0.37)


def test_sampled_rows_equal_full_batch():
    rng = _rng(99)
    rows, V = 50, 64
    x = rng.standard_normal((rows, V))
    t = rng.integers(0, V, rows)
    t[:7] = -100
    full = ce_forward(x, t, label_smoothing=0.1, lse_square_scale=1e-3, reduction="mean")
    summ = summarize_targets(t, V, reduction="mean")
    sel = np.array([3, 10, 49])
    part = rows_forward(x[sel], t[sel], V=V, alpha=summ.alpha, beta=summ.beta,
                        label_smoothing=0.1, lse_square_scale=1e-3)
    np.testing.assert_array_equal(part.grad, full.grad[sel])
    np.testing.assert_array_equal(part.ce, full.ce[sel])


def test_widen_bf16_bits_exact():
    rng = _rng(101)
    v = torch.tensor(rng.standard_normal(1000) * 5, dtype=torch.float32).to(torch.bfloat16)
    bits = v.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(widen(bits), v.double().numpy())


def test_argmax_uses_raw_logits_under_saturating_softcap():
    # tanh saturates to exactly 1.0 in float64 for both 100 and 101 at c = 1, so
    # the softcapped values tie while the raw logits do not: the raw maximum wins.
    x = np.array([[0.0, 100.0, 101.0, -3.0]])
    r = ce_forward(x, np.array([0]), softcap=1.0, reduction="none")
    assert np.tanh(100.0) == np.tanh(101.0)
    assert r.argmax[0] == 2


# ---------------------------------------------------------------------------
# The tolerance helper: the per-element magnitude M of the gradient's terms
# (it sizes every bf16 gradient bar), pinned to hand-derived values.
# ---------------------------------------------------------------------------

HELPERS = os.path.join(os.path.dirname(__file__), "golden", "tolerance_helpers.json")


def _helper_cases():
    with open(HELPERS) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _helper_cases()["mag_cases"], ids=lambda c: c["name"])
def test_gradient_magnitude_helper_golden(case):
    x = np.array([[_eval(e) for e in case["x_expr"]]])
    t = np.array([case["target"]])
    w = np.array(case["weight"]) if "weight" in case else None
    summ = summarize_targets(t, x.shape[1], -100, w, case["reduction"])
    r = rows_forward(x, t, V=x.shape[1], alpha=summ.alpha, beta=summ.beta, weight=w,
                     label_smoothing=case.get("label_smoothing", 0.0),
                     lse_square_scale=case.get("lse_square_scale", 0.0),
                     softcap=case.get("softcap"), want_grad=True, want_mag=True)
    want = np.array([_eval(e) for e in case["mag"]])
    np.testing.assert_allclose(r.mag[0], want, rtol=1e-12, atol=0)
    # M bounds the gradient it describes (triangle inequality), elementwise
    assert np.all(np.abs(r.grad[0]) <= r.mag[0] * (1 + 1e-12))


def test_gradient_magnitude_helper_rows_not_counted():
    """Ignored and out-of-range rows have no gradient terms: M is 0 there."""
    x = np.array([[0.0, 1.0, 2.0]] * 3)
    t = np.array([-100, 7, 1])
    summ = summarize_targets(t, 3, -100, None, "mean")
    r = rows_forward(x, t, V=3, alpha=summ.alpha, beta=summ.beta, want_grad=True,
                     want_mag=True)
    assert np.all(r.mag[:2] == 0.0)
    assert np.all(r.mag[2] > 0.0)


def _argmax_nan_first(row):
    """Brute force: a NaN ranks above every number, then the largest value;
    the lowest index wins ties."""
    best = None
    for k, v in enumerate(row):
        if best is None:
            best = k
            continue
        b = row[best]
        if math.isnan(b):
            continue
        if math.isnan(v) or v > b:
            best = k
    return best


def test_argmax_nan_and_inf_convention():
    g = _rng(77)
    x = g.integers(-3, 4, size=(40, 9)).astype(np.float64)
    for r in range(0, 40, 2):
        x[r, g.integers(0, 9)] = np.nan
    for r in range(1, 40, 4):
        x[r, g.integers(0, 9)] = np.inf
    x[3, :] = np.nan
    x[5, 2] = np.nan
    x[5, 6] = np.nan
    t = g.integers(0, 9, size=40)
    r = ce_forward(x, t, reduction="none")
    want = np.array([_argmax_nan_first(row) for row in x])
    np.testing.assert_array_equal(r.argmax, want)
    # torch orders NaN the same way (first occurrence)
    np.testing.assert_array_equal(torch.argmax(torch.from_numpy(x), dim=1).numpy(), want)
    bad = np.isnan(x).any(1) | np.isposinf(x).any(1)
    assert np.all(np.isnan(r.loss[bad])) and np.all(np.isfinite(r.loss[~bad]))
    assert np.all(np.isnan(r.grad[bad])) and np.all(np.isfinite(r.grad[~bad]))


def test_minus_inf_logit_without_smoothing_matches_torch():
    """A -inf logit away from the target: without smoothing the loss is
    -log p_y (finite) and the gradient finite, as torch computes it; with
    smoothing the term eps/V * log p_k of that class is +inf."""
    x = np.array([[0.5, -np.inf, 2.0, -1.0], [1.0, 0.0, -np.inf, 3.0]])
    t = np.array([2, 3])
    r = ce_forward(x, t, reduction="none")
    want = torch.nn.functional.cross_entropy(torch.from_numpy(x), torch.from_numpy(t),
                                             reduction="none").numpy()
    np.testing.assert_allclose(r.loss, want, rtol=1e-14)
    xt = torch.from_numpy(x).requires_grad_(True)
    torch.nn.functional.cross_entropy(xt, torch.from_numpy(t), reduction="sum").backward()
    np.testing.assert_allclose(r.grad, xt.grad.numpy(), rtol=1e-14, atol=1e-300)
    rs = ce_forward(x, t, label_smoothing=0.1, reduction="none")
    assert np.all(np.isposinf(rs.loss))
