"""GPU parity of the linear layer fused with the cross-entropy
(ce_linear_forward through the C ABI) against the float64 oracle
(oracle/linear_oracle.py).

Tolerances, derived from the arithmetic of the HIP path (bf16 inputs, fp32
products and cross-entropy, G rounded to bf16 before the gradient products):
  * logits: |dz_ik| <= H 2^-24 (|hidden| @ |weight|^T)_ik (fp32 accumulation
    of exact bf16 products), so a row's loss moves by at most 2 max_k dz_ik
    (its log-sum-exp and its target logit), plus the cross-entropy's own
    1e-5 relative bar;
  * gradients: G rounded to bf16 moves each term of d hidden = G @ weight
    and d weight = G^T @ hidden by at most 2^-9 of its magnitude, and the
    fp32 sums add at most K 2^-24 of it, so |error| <= (2^-8 + K 2^-24) M
    with M = |G| @ |weight| (resp. |G|^T @ |hidden|), plus 1e-7.
Where the two largest logits of a row are closer than their error bound
the argmax may pick either; it must then be one of the candidates.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import grad_magnitudes, linear_forward
from softmax_cross_entropy_amd import linear_cross_entropy, linear_forward_raw
from softmax_cross_entropy_amd._lib import CE_F_FORCE_FUSED, CE_F_SHAPE_ALT

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(**kw):
    print("CASE " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _bits(a: torch.Tensor) -> np.ndarray:
    return a.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _make(rows, H, V, seed, n_ignored):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(rows, H, generator=g) * 0.5).to(torch.bfloat16)
    w = (torch.randn(V, H, generator=g) * (2.0 / H ** 0.5)).to(torch.bfloat16)
    t = synth.make_targets(rows, V, seed, n_ignored)
    return x, w, t


def _check(x, w, t, res, *, cw=None, eps=0.0, lam=0.0, softcap=None, reduction="mean",
           grad_scale=None, what=""):
    loss, zl, acc, am, cnt, gh, gw = res
    rows, H = x.shape
    V = w.shape[0]
    ref = linear_forward(_bits(x), _bits(w), t.numpy(),
                         class_weight=None if cw is None else cw.numpy(), label_smoothing=eps,
                         lse_square_scale=lam, softcap=softcap, reduction=reduction)
    r = ref.ce
    counted = (t.numpy() != -100)
    # logits error bound per row, and the loss bound it implies: the row's
    # log-sum-exp and target logit each move by at most dz; the z-loss
    # lam lse^2 by at most 2 lam |lse| dz with |lse| <= max |z| + ln V
    dz = H * 2.0 ** -24 * ref.logits_abs.max(axis=1)
    row_bound = 2.0 * dz
    if lam > 0.0:
        lse_max = np.abs(ref.logits).max(axis=1) + np.log(V)
        row_bound = row_bound + 2.0 * lam * lse_max * dz
    row_bound = np.where(counted, row_bound, 0.0)
    if reduction == "none":
        got = loss.cpu().double().numpy()
        want = np.asarray(r.loss, dtype=np.float64)
        tol = 1e-5 * np.abs(want) + row_bound + 1e-7
        assert np.all(np.abs(got - want) <= tol), (what, np.max(np.abs(got - want) - tol))
    else:
        scale = 1.0 / r.D if reduction == "mean" else 1.0
        want = float(r.loss)
        tol = 1e-5 * abs(want) + scale * row_bound.sum() + 1e-7
        assert abs(loss.item() - want) <= tol, (what, loss.item(), want, tol)
    # argmax: exact where the top two logits are farther apart than the bound
    srt = np.sort(ref.logits, axis=1)
    gap = srt[:, -1] - srt[:, -2] if V > 1 else np.full(rows, np.inf)
    am_g = am.cpu().numpy()
    for i in range(rows):
        if not counted[i]:
            assert am_g[i] == -1
        elif gap[i] > 2.0 * dz[i]:
            assert am_g[i] == r.argmax[i], (what, i)
        else:
            assert ref.logits[i, am_g[i]] >= srt[i, -1] - 2.0 * dz[i], (what, i)
    c = cnt.cpu().numpy()
    assert int(c[0]) == r.n_valid
    assert int(c[1]) == int(np.sum((am_g == t.numpy()) & counted))
    if gh is None:
        return
    G = r.grad if grad_scale is None else r.grad * np.asarray(grad_scale).reshape(-1, 1)
    m_h, m_w = grad_magnitudes(_bits(x), _bits(w), G)
    xf = (_bits(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (_bits(w).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want_h = G @ wf
    want_w = G.T @ xf
    got_h = gh.cpu().double().numpy()
    got_w = gw.cpu().double().numpy()
    tol_h = (2.0 ** -8 + V * 2.0 ** -24) * m_h + 1e-7
    tol_w = (2.0 ** -8 + rows * 2.0 ** -24) * m_w + 1e-7
    eh = np.abs(got_h - want_h) - tol_h
    ew = np.abs(got_w - want_w) - tol_w
    assert np.all(eh <= 0), (what, "grad_hidden", float(eh.max()))
    assert np.all(ew <= 0), (what, "grad_weight", float(ew.max()))
    assert np.all(got_h[~counted] == 0.0), (what, "ignored rows")


OPTS = {
    "plain": dict(),
    "smooth_weight": dict(eps=0.1, cw=True),
    "softcap_zloss": dict(softcap=5.0, lam=1e-3),
    "all": dict(eps=0.2, cw=True, softcap=3.0, lam=1e-2),
}


@pytest.mark.parametrize("opt", list(OPTS))
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
# The first three shapes take the row kernel on the chunk's fp32 logits (the
# gradient narrowed to bf16 by its own kernel); the last three take split
# rows, whose kernel writes the bf16 gradient itself: a row pair of 5000
# vectors, a ragged row pair of 10000 vectors + 3 in three chunks (the last
# partial), and quarter rows of 17500 vectors + 1. Chunks this small would
# take split-V; CE_F_FORCE_FUSED keeps them on the split-row kernels, which
# chunks of 256 rows and more take by themselves.
@pytest.mark.parametrize("shape,chunk,flags", [((37, 64, 3001), 0, 0), ((300, 96, 4096), 64, 0),
                                               ((130, 128, 8000), 29, 0),
                                               ((40, 32, 20000), 0, CE_F_FORCE_FUSED),
                                               ((33, 32, 40003), 16, CE_F_FORCE_FUSED),
                                               ((24, 32, 70001), 0, CE_F_FORCE_FUSED)])
def test_linear_parity(opt, reduction, shape, chunk, flags):
    rows, H, V = shape
    o = OPTS[opt]
    x, w, t = _make(rows, H, V, rows + V, rows // 6)
    cw = (0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(V))
          if o.get("cw") else None)
    _announce(name="linear", rows=rows, H=H, V=V, chunk=chunk, opt=opt, reduction=reduction)
    res = linear_forward_raw(x.to(DEV), w.to(DEV), t.to(DEV),
                             None if cw is None else cw.to(DEV), -100, o.get("eps", 0.0),
                             o.get("lam", 0.0), o.get("softcap"), reduction, grad=True,
                             z_loss=True, token_accuracy=True, argmax=True, counts=True,
                             chunk_rows=chunk, flags=flags)
    torch.cuda.synchronize()
    _check(x, w, t, res, cw=cw, eps=o.get("eps", 0.0), lam=o.get("lam", 0.0),
           softcap=o.get("softcap"), reduction=reduction, what=f"{opt}/{reduction}/{shape}")


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("shape,chunk", [((40, 32, 20000), 0), ((33, 32, 40003), 16)])
def test_linear_auto_splitv(reduction, shape, chunk):
    """Chunks of fewer than 256 rows of more than 4096 vectors take the
    split-V path on their own (no test hook), every option on."""
    from softmax_cross_entropy_amd import _lib
    rows, H, V = shape
    o = OPTS["all"]
    cr = chunk or rows
    ldl = (V + 3) // 4 * 4
    plan = _lib.ce_plan_path(1 << 20, _lib.CE_F32, cr, V, ldl, 1 << 20, o["eps"], 0)
    assert _lib.PATH_NAMES[plan] == "splitv"
    x, w, t = _make(rows, H, V, rows + V + 1, rows // 6)
    cw = 0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(V + 1))
    _announce(name="linear-auto-splitv", rows=rows, H=H, V=V, chunk=chunk, reduction=reduction)
    res = linear_forward_raw(x.to(DEV), w.to(DEV), t.to(DEV), cw.to(DEV), -100, o["eps"],
                             o["lam"], o["softcap"], reduction, grad=True, z_loss=True,
                             token_accuracy=True, argmax=True, counts=True, chunk_rows=chunk,
                             flags=0)
    torch.cuda.synchronize()
    _check(x, w, t, res, cw=cw, eps=o["eps"], lam=o["lam"], softcap=o["softcap"],
           reduction=reduction, what=f"auto-splitv/{reduction}/{shape}")


@pytest.mark.parametrize("rows,V,chunk", [(64, 5000, 24), (600, 20000, 300)])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_linear_autograd_grad_output(reduction, rows, V, chunk):
    """loss.backward(grad_output): mean scales the forward's gradients; none
    recomputes them with the per-row grad_output (600 x 20000: two chunks of
    300 rows on the split-row kernel, which applies each row's value before
    it rounds the gradient to bf16)."""
    H = 64
    x, w, t = _make(rows, H, V, 77, 8)
    _announce(name="linear-autograd", rows=rows, H=H, V=V, reduction=reduction)
    xd = x.to(DEV).requires_grad_(True)
    wd = w.to(DEV).requires_grad_(True)
    out = linear_cross_entropy(xd, wd, t.to(DEV), label_smoothing=0.1, reduction=reduction,
                               chunk_rows=chunk)
    if reduction == "none":
        go = torch.linspace(0.5, 2.0, rows)
        out.loss.backward(go.to(DEV))
        scale = go.double().numpy()
    else:
        out.loss.backward(torch.tensor(2.5, device=DEV))
        scale = np.full(rows, 2.5)
    torch.cuda.synchronize()
    ref = linear_forward(_bits(x), _bits(w), t.numpy(), label_smoothing=0.1, reduction=reduction)
    G = ref.ce.grad * scale.reshape(-1, 1)
    m_h, m_w = grad_magnitudes(_bits(x), _bits(w), G)
    xf = (_bits(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (_bits(w).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # the returned gradients are rounded to the parameters' dtype (bf16)
    gh = xd.grad.double().cpu().numpy()
    gw = wd.grad.double().cpu().numpy()
    want_h, want_w = G @ wf, G.T @ xf
    tol_h = (2.0 ** -7 + V * 2.0 ** -24) * m_h + np.abs(want_h) * 2.0 ** -8 + 1e-7
    tol_w = (2.0 ** -7 + rows * 2.0 ** -24) * m_w + np.abs(want_w) * 2.0 ** -8 + 1e-7
    assert np.all(np.abs(gh - want_h) <= tol_h)
    assert np.all(np.abs(gw - want_w) <= tol_w)


def test_linear_all_ignored_and_empty():
    rows, H, V = 16, 32, 1000
    x, w, _ = _make(rows, H, V, 5, 0)
    t = torch.full((rows,), -100, dtype=torch.int64)
    _announce(name="linear-all-ignored", rows=rows)
    loss, _, _, _, cnt, gh, gw = linear_forward_raw(x.to(DEV), w.to(DEV), t.to(DEV), counts=True)
    torch.cuda.synchronize()
    assert torch.isnan(loss).item()
    assert int(cnt[0]) == 0
    assert torch.count_nonzero(gh).item() == 0 and torch.count_nonzero(gw).item() == 0
    _announce(name="linear-empty", rows=0)
    loss, _, _, _, cnt, gh, gw = linear_forward_raw(
        x[:0].to(DEV), w.to(DEV), t[:0].to(DEV), counts=True)
    torch.cuda.synchronize()
    assert torch.isnan(loss).item() and int(cnt[0]) == 0
    assert gh.numel() == 0 and torch.count_nonzero(gw).item() == 0


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_linear_alt_layout(reduction):
    """Quarter-row sizes on the alternative layout (a pair of 1024-thread
    workgroups per row), every option on."""
    rows, H, V = 20, 32, 70001
    x, w, t = _make(rows, H, V, 71, 3)
    cw = 0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(3))
    _announce(name="linear-alt", rows=rows, H=H, V=V, reduction=reduction)
    res = linear_forward_raw(x.to(DEV), w.to(DEV), t.to(DEV), cw.to(DEV), -100, 0.2, 1e-2, 3.0,
                             reduction, grad=True, z_loss=True, token_accuracy=True,
                             argmax=True, counts=True,
                             flags=CE_F_FORCE_FUSED | CE_F_SHAPE_ALT)
    torch.cuda.synchronize()
    _check(x, w, t, res, cw=cw, eps=0.2, lam=1e-2, softcap=3.0, reduction=reduction,
           what=f"alt/{reduction}")


@pytest.mark.parametrize("V", [3001, 20000])
def test_linear_target_out_of_range(V):
    """A target outside [0, V) that is not ignore_index: that row's loss is
    NaN and its gradient zero (V = 20000: zeros written as bf16 by the
    split-row kernel); every other value equals, bit for bit, the call with
    that row ignored, which is checked against the oracle."""
    rows, H = 40, 32
    x, w, t = _make(rows, H, V, 211, 5)
    bad = t.clone()
    bad[7] = V + 5
    ign = t.clone()
    ign[7] = -100
    _announce(name="linear-target-range", rows=rows, H=H, V=V)
    kw = dict(reduction="none", grad=True, z_loss=True, token_accuracy=True, argmax=True,
              counts=True, chunk_rows=16, flags=CE_F_FORCE_FUSED)
    rb = linear_forward_raw(x.to(DEV), w.to(DEV), bad.to(DEV), **kw)
    ri = linear_forward_raw(x.to(DEV), w.to(DEV), ign.to(DEV), **kw)
    torch.cuda.synchronize()
    lb, li = rb[0].cpu(), ri[0].cpu()
    assert torch.isnan(lb[7]).item() and li[7].item() == 0.0
    keep = torch.arange(rows) != 7
    assert torch.equal(lb[keep], li[keep])
    assert torch.equal(rb[3].cpu(), ri[3].cpu())  # argmax (-1 on both rows)
    assert torch.equal(rb[5], ri[5]) and torch.equal(rb[6], ri[6])  # both gradients
    assert torch.count_nonzero(rb[5][7]).item() == 0
    assert torch.equal(rb[4].cpu(), ri[4].cpu())  # counts: neither row is counted
    _check(x, w, ign, ri, reduction="none", what=f"target-range/{V}")


def test_linear_medium_default_chunk():
    """512 x 1024 hidden, V = 32000 (one default chunk), mean, every output."""
    rows, H, V = 512, 1024, 32000
    x, w, t = _make(rows, H, V, 123, 25)
    _announce(name="linear-medium", rows=rows, H=H, V=V)
    res = linear_forward_raw(x.to(DEV), w.to(DEV), t.to(DEV), label_smoothing=0.1,
                             lse_square_scale=1e-4, z_loss=True, token_accuracy=True,
                             argmax=True, counts=True)
    torch.cuda.synchronize()
    _check(x, w, t, res, eps=0.1, lam=1e-4, what="medium")


def test_linear_dirty_workspace_and_default_chunks():
    """The workspace may hold anything: every call clears what it needs. 2100
    rows take two default chunks (2048 + 52); calls on a workspace filled with
    0xFF bytes, and again after a refill, give the bits of a call on a zeroed
    one, and the oracle's values."""
    from softmax_cross_entropy_amd import _lib
    rows, H, V = 2100, 256, 4000
    x, w, t = _make(rows, H, V, 321, 40)
    _announce(name="linear-dirty-workspace", rows=rows, H=H, V=V)
    xd, wd, td = x.to(DEV), w.to(DEV), t.to(DEV)
    nbytes = _lib.ce_linear_workspace_bytes(rows, H, V, 0, 0)
    s = torch.cuda.current_stream().cuda_stream
    outs = []
    for fill in (0x00, 0xFF, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        loss = torch.empty((), device=DEV)
        am = torch.empty((rows,), dtype=torch.int64, device=DEV)
        cnt = torch.empty((2,), dtype=torch.int64, device=DEV)
        gh = torch.empty((rows, H), device=DEV)
        gw = torch.empty((V, H), device=DEV)
        st = _lib.ce_linear_forward(xd.data_ptr(), H, wd.data_ptr(), H, _lib.CE_BF16, rows, H, V,
                                    td.data_ptr(), 0, -100, 0.1, 1e-4, 0.0, _lib.CE_RED_MEAN, 0,
                                    0, 0, 0, loss.data_ptr(), 0, 0, am.data_ptr(), cnt.data_ptr(),
                                    gh.data_ptr(), H, gw.data_ptr(), H, ws.data_ptr(), nbytes, s)
        assert st == 0, _lib.ce_status_string(st)
        torch.cuda.synchronize()
        outs.append((loss, am, cnt, gh, gw))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b)
    loss, am, cnt, gh, gw = outs[0]
    _check(x, w, t, (loss, None, None, am, cnt, gh, gw), eps=0.1, lam=1e-4,
           what="dirty-workspace")


def test_linear_bench_shape_sampled():
    """The benchmark's batch: 4096 x 4096 hidden, V = 128256, mean, default
    chunks, both gradients. Every row's loss term, argmax and the counts
    against the oracle (evaluated in row blocks: oracle.linear_forward_rows),
    d loss / d hidden on 16 sampled rows and d loss / d weight on 16 sampled
    classes, to the tolerances of _check."""
    from oracle import linear_forward_rows
    rows, H, V = 4096, 4096, 128256
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    x = (torch.randn(rows, H, device=DEV, generator=g) * 0.5).to(torch.bfloat16)
    w = (torch.randn(V, H, device=DEV, generator=g) * (2.0 / H ** 0.5)).to(torch.bfloat16)
    t = synth.make_targets(rows, V, 7, rows // 20)
    _announce(name="linear-bench-shape", rows=rows, H=H, V=V)
    loss, _, acc, am, cnt, gh, gw = linear_forward_raw(x, w, t.to(DEV), token_accuracy=True,
                                                       argmax=True, counts=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    counted = t.numpy() != -100
    sr = np.sort(np.concatenate([[0, rows - 1], rng.choice(np.nonzero(counted)[0], 13,
                                                           replace=False),
                                 np.nonzero(~counted)[0][:1]]))
    sc = np.sort(np.concatenate([[0, V - 1], rng.choice(V, 14, replace=False)]))
    am_g = am.cpu().numpy()
    xb, wb = _bits(x), _bits(w)
    print("  gpu done; oracle over every row in blocks", flush=True)
    ref = linear_forward_rows(xb, wb, t.numpy(), sample_rows=sr, sample_cols=sc, at_cols=am_g)
    # loss: the fp32 logits move by at most dz per row, the row's loss by 2 dz
    dz = H * 2.0 ** -24 * ref.logits_abs_max
    tol = 1e-5 * abs(ref.loss) + (2.0 * dz[counted]).sum() / ref.D + 1e-7
    assert abs(loss.item() - ref.loss) <= tol, (loss.item(), ref.loss, tol)
    # argmax: exact where the top two logits are farther apart than the bound
    gap = ref.top2[:, 0] - ref.top2[:, 1]
    exact = counted & (gap > 2.0 * dz)
    np.testing.assert_array_equal(am_g[exact], ref.argmax[exact])
    near = counted & ~exact
    assert np.all(ref.at_cols[near] >= ref.top2[near, 0] - 2.0 * dz[near])
    assert np.all(am_g[~counted] == -1)
    c = cnt.cpu().numpy()
    assert int(c[0]) == ref.n_valid
    assert int(c[1]) == int(np.sum((am_g == t.numpy()) & counted))
    assert abs(acc.item() - np.float32(c[1] / c[0])) <= 1e-7
    got_h = gh[torch.from_numpy(sr).to(DEV)].double().cpu().numpy()
    got_w = gw[torch.from_numpy(sc).to(DEV)].double().cpu().numpy()
    tol_h = (2.0 ** -8 + V * 2.0 ** -24) * ref.mag_hidden + 1e-7
    tol_w = (2.0 ** -8 + rows * 2.0 ** -24) * ref.mag_weight + 1e-7
    eh = np.abs(got_h - ref.grad_hidden) - tol_h
    ew = np.abs(got_w - ref.grad_weight) - tol_w
    assert np.all(eh <= 0), ("grad_hidden", float(eh.max()))
    assert np.all(ew <= 0), ("grad_weight", float(ew.max()))


# The forward without gradients on the matrix-core kernel (CE_F_LINEAR_ON_CHIP:
# partials of 256-class blocks, logits kept on chip) and on the default
# library GEMM path with fp32 logits. Shapes: ragged classes (V not a
# multiple of 256), rows not a multiple of 128, H not a multiple of 64, and
# one row block spanning several XCD patches.
FWD_SHAPES = [(37, 64, 3001), (300, 96, 4096), (130, 136, 8000), (33, 32, 40003),
              (1030, 128, 2304)]


@pytest.mark.parametrize("opt", list(OPTS))
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("shape", FWD_SHAPES)
def test_linear_forward_only_matrix_core(opt, reduction, shape):
    from softmax_cross_entropy_amd._lib import CE_F_LINEAR_ON_CHIP
    rows, H, V = shape
    o = OPTS[opt]
    x, w, t = _make(rows, H, V, 900 + rows + V, max(1, rows // 12))
    cw = (0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(V))
          if o.get("cw") else None)
    _announce(name="linear-forward-only", rows=rows, H=H, V=V, opt=opt, reduction=reduction)
    kw = dict(class_weight=None if cw is None else cw.to(DEV), label_smoothing=o.get("eps", 0.0),
              lse_square_scale=o.get("lam", 0.0), softcap=o.get("softcap"), reduction=reduction,
              grad=False, z_loss=True, token_accuracy=True, argmax=True, counts=True)
    res = linear_forward_raw(x.to(DEV), w.to(DEV), t.to(DEV), flags=CE_F_LINEAR_ON_CHIP, **kw)
    lib = linear_forward_raw(x.to(DEV), w.to(DEV), t.to(DEV), **kw)
    torch.cuda.synchronize()
    _check(x, w, t, res, cw=cw, eps=o.get("eps", 0.0), lam=o.get("lam", 0.0),
           softcap=o.get("softcap"), reduction=reduction, what=f"forward-only/{opt}")
    _check(x, w, t, lib, cw=cw, eps=o.get("eps", 0.0), lam=o.get("lam", 0.0),
           softcap=o.get("softcap"), reduction=reduction, what=f"forward-only-library/{opt}")
