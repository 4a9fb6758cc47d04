"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case prints its name, shape, dtype, options and kernel path before it
touches the GPU. Every case compares every row's loss terms, argmax, counts
and accuracy with the oracle; small and medium cases compare every gradient
element, and the full-size workloads (run in the benchmark's launch
configuration, automatic path) compare every row's gradient except at
16384 x 262144, where a seeded sample of rows is compared.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import synth
from oracle import reduce_rows
from parity import (OracleRef, assert_acc_exact, assert_grad_close, assert_loss_close,
                    host_logits, oracle_rows)
from softmax_cross_entropy_amd import _lib, backward_, backward_recompute, forward_raw
from softmax_cross_entropy_amd._lib import (CE_F_EXCHANGE_ONE_POLL, CE_F_FORCE_FUSED,
                                            CE_F_FORCE_SCALAR, CE_F_FORCE_SPLITV,
                                            CE_F_SHAPE_ALT)

pytestmark = pytest.mark.gpu

DEV = "cuda"
PATH_FLAGS = {"auto": 0, "fused": CE_F_FORCE_FUSED, "splitv": CE_F_FORCE_SPLITV,
              "scalar": CE_F_FORCE_SCALAR, "fused_alt": CE_F_FORCE_FUSED | CE_F_SHAPE_ALT}


def _announce(**kw):
    print("CASE " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _padded(x_cpu: torch.Tensor, stride: int) -> torch.Tensor:
    """(rows, V) tensor on the GPU inside a (rows, stride) buffer."""
    rows, V = x_cpu.shape
    buf = torch.full((rows, stride), float("nan"), dtype=x_cpu.dtype, device=DEV)
    buf[:, :V].copy_(x_cpu.to(DEV))
    return buf[:, :V]


def _plan(x, weight, eps, flags):
    rows, V = x.shape
    return _lib.PATH_NAMES.get(_lib.ce_plan_path(
        x.data_ptr(), _lib.dtype_code(x.dtype), rows, V, x.stride(0),
        0 if weight is None else weight.data_ptr(), eps, flags), "?")


def run_case(x_cpu, t_cpu, *, weight=None, ignore_index=-100, eps=0.0, lam=0.0, softcap=None,
             reduction="mean", path="auto", stride=None, name=""):
    """Run GPU + oracle on the same inputs and compare every output."""
    rows, V = x_cpu.shape
    stride = V if stride is None else stride
    x = _padded(x_cpu, stride)
    t = t_cpu.to(DEV)
    w = None if weight is None else weight.to(DEV)
    flags = PATH_FLAGS[path]
    _announce(name=name, rows=rows, V=V, stride=stride, dtype=x.dtype, eps=eps, lam=lam,
              softcap=softcap, weight=weight is not None, reduction=reduction, path=path,
              plan=_plan(x, w, eps, flags))
    xh = host_logits(x_cpu)
    loss, z, acc, arg, counts = forward_raw(
        x, t, w, ignore_index, eps, lam, softcap, reduction, grad=True, z_loss=True,
        token_accuracy=True, argmax=True, counts=True, flags=flags)
    torch.cuda.synchronize()
    ref = OracleRef(xh, t_cpu.numpy(), weight=None if weight is None else weight.numpy(),
                    ignore_index=ignore_index, label_smoothing=eps, lse_square_scale=lam,
                    softcap=softcap, reduction=reduction)
    assert_loss_close(loss.cpu().numpy(), ref.loss, "loss")
    assert_loss_close(z.cpu().numpy(), ref.z_loss, "z_loss")
    np.testing.assert_array_equal(arg.cpu().numpy(), ref.argmax)
    c = counts.cpu().numpy()
    assert int(c[0]) == ref.summ.n and int(c[1]) == ref.n_correct
    if reduction == "none":
        np.testing.assert_array_equal(acc.cpu().numpy(), ref.acc.astype(np.float32))
    else:
        assert_acc_exact(acc.item(), ref.n_correct, ref.summ.n)
    assert_grad_close(x, ref.grad, ref.mag, zero_rows=ref.not_counted)
    if stride > V:  # padding columns untouched
        pad = x.as_strided((rows, stride - V), (stride, 1), x.storage_offset() + V)
        assert torch.isnan(pad.float()).all()
    return x, ref


# ---------------------------------------------------------------------------
# The 64 x 4096 fp32 workload, every path and reduction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["auto", "fused", "splitv", "scalar"])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_small_workload(path, reduction):
    w = synth.WORKLOADS["ce_64x4096_f32"]
    inp = synth.make_inputs(w, "cpu")
    run_case(inp.logits, inp.target, reduction=reduction, path=path, name=w.name)


# ---------------------------------------------------------------------------
# Options x dtype x path, ragged rows (V not a multiple of a vector)
# ---------------------------------------------------------------------------

OPTS = {
    "plain": dict(),
    "weight": dict(weight=True),
    "smooth": dict(eps=0.1),
    "weight_smooth": dict(weight=True, eps=0.2),
    "softcap": dict(softcap=5.0),
    "zloss": dict(lam=1e-3),
    "all": dict(weight=True, eps=0.1, softcap=4.0, lam=1e-2),
}


@pytest.mark.parametrize("opt", list(OPTS))
@pytest.mark.parametrize("path", ["fused", "splitv", "scalar"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_options_matrix(opt, path, dtype, reduction):
    o = OPTS[opt]
    rows, V = 37, 3001
    x = synth.make_logits(rows, V, dtype, 3.0, 7)
    t = synth.make_targets(rows, V, 7, 4)
    wt = None
    if o.get("weight"):
        wt = 0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(9))
    run_case(x, t, weight=wt, eps=o.get("eps", 0.0), lam=o.get("lam", 0.0),
             softcap=o.get("softcap"), reduction=reduction, path=path, stride=3008,
             name=f"opts-{opt}")


@pytest.mark.parametrize("V", [1, 2, 3, 17, 4099, 8192])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("pad", [False, True])
@pytest.mark.parametrize("rows", [1, 7])
def test_edge_sizes(V, dtype, pad, rows):
    x = synth.make_logits(rows, V, dtype, 2.0, 11 + V)
    t = synth.make_targets(rows, V, 11 + V, 1 if rows > 1 else 0)
    stride = (V + 7) // 8 * 8 + (8 if pad else 0) if pad else V
    run_case(x, t, eps=0.05, lam=1e-3, reduction="mean", stride=stride, name="edge")
    run_case(x, t, reduction="none", stride=stride, name="edge-none")


def test_ignore_index_is_a_real_class():
    rows, V = 50, 512
    x = synth.make_logits(rows, V, torch.float32, 1.0, 21)
    t = synth.make_targets(rows, V, 21, 0)
    t[::3] = 5
    run_case(x, t, ignore_index=5, reduction="mean", name="ignore5")


def test_ties_in_argmax_bf16():
    rows, V = 64, 2048
    x = torch.randint(-3, 3, (rows, V), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    t = synth.make_targets(rows, V, 3, 0)
    for path in ("fused", "splitv", "scalar"):
        run_case(x, t, reduction="none", path=path, name="ties")


def test_large_logit_spikes_exact_zero_loss():
    rows, V = 16, 4096
    x = synth.make_logits(rows, V, torch.float32, 1.0, 31)
    t = synth.make_targets(rows, V, 31, 0)
    for r in range(0, rows, 2):
        x[r, t[r]] = 80.0
    for r in range(1, rows, 2):
        x[r, (int(t[r]) + 7) % V] = 80.0
    for path in ("fused", "splitv", "scalar"):
        _, ref = run_case(x, t, reduction="none", path=path, name="spikes")
        assert np.all(ref.ce[::2] == 0.0)


# ---------------------------------------------------------------------------
# Ignored rows, all-ignored batches, targets out of range
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["auto", "fused", "splitv", "scalar"])
def test_all_ignored_nonfinite_small(path):
    rows, V = 64, 1024
    x = synth.make_logits(rows, V, torch.bfloat16, 1.0, 41)
    x[0::4] = float("nan")
    x[1::4] = float("inf")
    x[2::4] = float("-inf")
    t = torch.full((rows,), -100, dtype=torch.int64)
    _announce(name="all-ignored-small", path=path)
    xd = x.to(DEV)
    loss, z, acc, arg, counts = forward_raw(xd, t.to(DEV), lse_square_scale=1e-4, z_loss=True,
                                            token_accuracy=True, argmax=True, counts=True,
                                            flags=PATH_FLAGS[path])
    torch.cuda.synchronize()
    assert math.isnan(loss.item()) and math.isnan(z.item()) and math.isnan(acc.item())
    assert counts.tolist() == [0, 0]
    assert (arg == -1).all()
    assert (xd.view(torch.int16) == 0).all()


def test_all_ignored_full_size():
    w = synth.WORKLOADS["ce_512x262144_bf16_allignored"]
    _announce(name=w.name, rows=w.rows, V=w.V)
    inp = synth.make_inputs(w, DEV)
    loss, z, acc, arg, counts = forward_raw(inp.logits, inp.target, z_loss=True,
                                            token_accuracy=True, argmax=True, counts=True)
    torch.cuda.synchronize()
    assert math.isnan(loss.item()) and math.isnan(z.item()) and math.isnan(acc.item())
    assert counts.tolist() == [0, 0]
    assert (inp.logits.view(torch.int16) == 0).all()
    s, _, _, _, _ = forward_raw(synth.make_inputs(w, DEV).logits, inp.target, reduction="sum")
    assert s.item() == 0.0


def test_bad_targets():
    rows, V = 8, 300
    x = synth.make_logits(rows, V, torch.float32, 1.0, 51)
    t = torch.tensor([0, 300, -1, -100, 5, 299, 1000, 7])
    run_case(x, t, reduction="none", name="bad-targets")
    run_case(x, t, reduction="mean", name="bad-targets-mean")
    _announce(name="bad-targets-check")
    with pytest.raises(_lib.CEError) as e:
        forward_raw(x.to(DEV), t.to(DEV), check_targets=True)
    assert e.value.status == _lib.CE_E_TARGET_RANGE
    ok = t.clone()
    ok[[1, 2, 6]] = 3
    forward_raw(x.to(DEV), ok.to(DEV), check_targets=True)


def test_zero_weight_mean():
    rows, V = 6, 40
    x = synth.make_logits(rows, V, torch.float32, 1.0, 53)
    t = torch.tensor([1, 2, 3, 1, 2, 3])
    w = torch.ones(V)
    w[1:4] = 0.0
    run_case(x, t, weight=w, reduction="mean", name="zero-weight")


def test_empty_batch():
    _announce(name="empty")
    x = torch.empty((0, 100), device=DEV)
    t = torch.empty((0,), dtype=torch.int64, device=DEV)
    loss, _, acc, _, counts = forward_raw(x, t, reduction="mean", token_accuracy=True, counts=True)
    assert math.isnan(loss.item()) and math.isnan(acc.item()) and counts.tolist() == [0, 0]
    loss, _, _, _, _ = forward_raw(x, t, reduction="sum")
    assert loss.item() == 0.0


# ---------------------------------------------------------------------------
# Backward (scale by grad_output), determinism, path cross-check
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("go", [1.0, 2.0, 0.37, "rows"])
@pytest.mark.parametrize("aligned", [True, False])
def test_backward_scale(dtype, go, aligned):
    rows, V = 33, 5003
    stride = 5008 if aligned else V
    x = synth.make_logits(rows, V, dtype, 2.0, 61)
    t = synth.make_targets(rows, V, 61, 3)
    red = "none" if go == "rows" else "mean"
    _announce(name="backward", dtype=dtype, go=go, aligned=aligned)
    xd = _padded(x, stride)
    forward_raw(xd, t.to(DEV), reduction=red)
    g0 = xd.detach().clone()
    if go == "rows":
        gov = torch.linspace(-2.0, 3.0, rows)
        gov[5] = 1.0
    else:
        gov = torch.tensor(go)
    backward_(xd, gov.to(DEV), per_row=(go == "rows"))
    torch.cuda.synchronize()
    # The backward is one multiply per element in float32, rounded to the dtype.
    want = (g0.float().cpu() * gov.float().reshape(-1, 1 if go == "rows" else 1)).to(dtype)
    assert torch.equal(xd.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       want.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


# ---------------------------------------------------------------------------
# Gradient recomputed from kept logits (ce_backward_recompute)
# ---------------------------------------------------------------------------

RECOMPUTE_OPTS = {
    "plain": dict(),
    "all": dict(weight=True, eps=0.1, softcap=4.0, lam=1e-2),
    "smooth_weight": dict(weight=True, eps=0.2),
}


@pytest.mark.parametrize("opt", list(RECOMPUTE_OPTS))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("reduction,go", [("mean", 1.0), ("sum", 2.5), ("none", "rows")])
@pytest.mark.parametrize("fwd_path,layout", [("fused", "aligned"), ("splitv", "aligned"),
                                             ("scalar", "unaligned"), ("fused", "inplace")])
def test_backward_recompute(opt, dtype, reduction, go, fwd_path, layout):
    o = RECOMPUTE_OPTS[opt]
    rows, V = 37, 3001
    stride = V if layout == "unaligned" else 3008
    x = synth.make_logits(rows, V, dtype, 3.0, 17)
    t = synth.make_targets(rows, V, 17, 4)
    t[3] = V + 5  # out of range: not counted, zero gradient
    wt = None
    if o.get("weight"):
        wt = 0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(19))
    _announce(name=f"recompute-{opt}", dtype=dtype, reduction=reduction, go=go, path=fwd_path,
              layout=layout)
    xd = _padded(x, stride)
    x_before = xd.detach().clone()
    td = t.to(DEV)
    wd = None if wt is None else wt.to(DEV)
    eps, lam, cap = o.get("eps", 0.0), o.get("lam", 0.0), o.get("softcap")
    stats = torch.empty((rows, 2), device=DEV, dtype=torch.float32)
    forward_raw(xd, td, wd, -100, eps, lam, cap, reduction, grad=False, row_stats=stats,
                flags=PATH_FLAGS[fwd_path])
    torch.cuda.synchronize()
    assert torch.equal(xd, x_before)  # a forward without the gradient only reads
    if go == "rows":
        gov = torch.linspace(-2.0, 3.0, rows)
    else:
        gov = torch.tensor(go)
    if layout == "inplace":
        g = backward_recompute(xd, td, wd, -100, eps, lam, cap, reduction, stats, gov.to(DEV),
                               grad=xd)
    else:
        g = backward_recompute(xd, td, wd, -100, eps, lam, cap, reduction, stats, gov.to(DEV))
        assert torch.equal(xd.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           x_before.cpu().view(torch.int16 if dtype == torch.bfloat16
                                               else torch.int32))
    torch.cuda.synchronize()
    ref = OracleRef(host_logits(x), t.numpy(), weight=None if wt is None else wt.numpy(),
                    label_smoothing=eps, lse_square_scale=lam, softcap=cap, reduction=reduction)
    scale = gov.double().numpy().reshape(-1, 1) if go == "rows" else float(go)
    assert_grad_close(g, ref.grad * scale, ref.mag * np.abs(scale), zero_rows=ref.not_counted)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_nograd_forward_claimed_rows_f32(reduction):
    """The forward without the gradient on fp32 rows of 12000 classes (the
    claimed-row kernel, 256 x 16 slots, more rows than workgroups, so rows
    follow one another on a workgroup): every scalar output against the
    oracle, and the logits untouched."""
    rows, V = 1600, 12000
    x = synth.make_logits(rows, V, torch.float32, 2.5, 41)
    t = synth.make_targets(rows, V, 41, rows // 10)
    _announce(name="nograd-claimed-f32", rows=rows, V=V, reduction=reduction)
    xd = x.to(DEV)
    x_before = xd.clone()
    loss, z, acc, arg, counts = forward_raw(xd, t.to(DEV), None, -100, 0.1, 1e-3, None, reduction,
                                            grad=False, z_loss=True, token_accuracy=True,
                                            argmax=True, counts=True)
    torch.cuda.synchronize()
    assert torch.equal(xd, x_before)
    ref = OracleRef(host_logits(x), t.numpy(), label_smoothing=0.1, lse_square_scale=1e-3,
                    reduction=reduction)
    assert_loss_close(loss.cpu().numpy(), ref.loss, "loss")
    assert_loss_close(z.cpu().numpy(), ref.z_loss, "z_loss")
    np.testing.assert_array_equal(arg.cpu().numpy(), ref.argmax)
    c = counts.cpu().numpy()
    assert int(c[0]) == ref.summ.n and int(c[1]) == ref.n_correct
    assert_acc_exact(acc.item(), ref.n_correct, ref.summ.n)


# ---------------------------------------------------------------------------
# The forward without the gradient on the split-row sizes: in the default
# layout each row streams through one workgroup (no exchange); the
# alternative layout keeps the split-row kernels. Every scalar output against
# the oracle, the logits untouched, and the kept per-row (m, log2 s) checked
# by recomputing the gradient from them.
# ---------------------------------------------------------------------------

NOGRAD_CASES = [
    # (dtype, V, rows, options); at least 256 rows (fewer take split-V)
    (torch.float32, 20001, 300, dict(weight=True, eps=0.1, softcap=15.0, lam=1e-3)),  # pair 512x8
    (torch.bfloat16, 40003, 300, dict()),                                             # pair 512x8
    (torch.float32, 50001, 300, dict(eps=0.05)),                                      # pair 512x16
    (torch.bfloat16, 131001, 280, dict(weight=True, eps=0.1, softcap=30.0, lam=1e-4)),
    (torch.float32, 128256, 300, dict(specials=True)),                                # quarters
    (torch.bfloat16, 262001, 260, dict(lam=1e-4, softcap=20.0, specials=True)),       # quarters
    (torch.float32, 128256, 300, dict(sigma=0.3, tie=1.5)),       # ties in the first and last chunk
]


@pytest.mark.parametrize("case", range(len(NOGRAD_CASES)))
@pytest.mark.parametrize("reduction", ["mean", "none"])
@pytest.mark.parametrize("layout", ["fused", "fused_alt"])
def test_nograd_streamed_rows(case, reduction, layout):
    dtype, V, rows, o = NOGRAD_CASES[case]
    seed = 900 + case
    x = synth.make_logits(rows, V, dtype, o.get("sigma", 2.5), seed)
    t = synth.make_targets(rows, V, seed, rows // 10)
    if o.get("tie"):
        for r in range(rows):
            x[r, V - 5] = o["tie"]
            if r % 2 == 0:
                x[r, 7 + r] = o["tie"]
        t[1::4] = V - 3
    if o.get("specials"):
        g = torch.Generator().manual_seed(seed)
        cols = lambda k: torch.randperm(V, generator=g)[:k].tolist()  # noqa: E731
        for r in range(0, rows, 7):
            kind = (r // 7) % 5
            if kind == 0:
                x[r, cols(1)[0]] = float("nan")
            elif kind == 1:  # a large logit before two NaNs
                c = sorted(cols(3))
                x[r, c[0]] = 50.0
                x[r, c[1]] = float("nan")
                x[r, c[2]] = float("nan")
            elif kind == 2:
                x[r, cols(1)[0]] = float("inf")
            elif kind == 3:
                x[r, V - 1] = float("nan")  # in the row tail
            else:
                x[r, cols(1)[0]] = float("-inf")
    t[5] = V + 3  # out of range: NaN loss, not counted, zero recomputed gradient
    wt = None
    if o.get("weight"):
        wt = 0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(seed))
    eps, lam, cap = o.get("eps", 0.0), o.get("lam", 0.0), o.get("softcap")
    stride = (V + 7) // 8 * 8
    xd = _padded(x, stride)
    x_before = xd.clone()
    td = t.to(DEV)
    wd = None if wt is None else wt.to(DEV)
    flags = PATH_FLAGS[layout]
    _announce(name=f"nograd-stream-{case}", rows=rows, V=V, dtype=dtype, reduction=reduction,
              layout=layout, plan=_plan(xd, wd, eps, flags))
    stats = torch.empty((rows, 2), device=DEV, dtype=torch.float32)
    loss, z, acc, arg, counts = forward_raw(xd, td, wd, -100, eps, lam, cap, reduction,
                                            grad=False, z_loss=True, token_accuracy=True,
                                            argmax=True, counts=True, row_stats=stats,
                                            flags=flags)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(xd.view(bits), x_before.view(bits))  # only read
    ref = OracleRef(host_logits(x), t.numpy(), weight=None if wt is None else wt.numpy(),
                    label_smoothing=eps, lse_square_scale=lam, softcap=cap, reduction=reduction)
    assert_loss_close(loss.cpu().numpy(), ref.loss, "loss")
    assert_loss_close(z.cpu().numpy(), ref.z_loss, "z_loss")
    np.testing.assert_array_equal(arg.cpu().numpy(), ref.argmax)
    c = counts.cpu().numpy()
    assert int(c[0]) == ref.summ.n and int(c[1]) == ref.n_correct
    if reduction == "none":
        np.testing.assert_array_equal(acc.cpu().numpy(), ref.acc.astype(np.float32))
    else:
        assert_acc_exact(acc.item(), ref.n_correct, ref.summ.n)
    go = torch.ones(rows) if reduction == "none" else torch.tensor(1.0)
    g = backward_recompute(xd, td, wd, -100, eps, lam, cap, reduction, stats, go.to(DEV))
    torch.cuda.synchronize()
    assert_grad_close(g, ref.grad, ref.mag, zero_rows=ref.not_counted)


def test_keep_logits_autograd_matches_inplace():
    import softmax_cross_entropy_amd as sce
    rows, V = 300, 8200
    x = synth.make_logits(rows, V, torch.bfloat16, 2.0, 23).to(DEV)
    t = synth.make_targets(rows, V, 23, 30).to(DEV)
    _announce(name="keep_logits", rows=rows, V=V)
    a = x.clone().requires_grad_(True)
    la = sce.cross_entropy(a, t, label_smoothing=0.1, lse_square_scale=1e-3, keep_logits=True)
    (la * 3.0).backward()
    b = x.clone().requires_grad_(True)
    lb = sce.cross_entropy(b, t, label_smoothing=0.1, lse_square_scale=1e-3, inplace=False)
    (lb * 3.0).backward()
    torch.cuda.synchronize()
    assert torch.equal(a.detach(), x)          # logits kept
    assert la.item() == lb.item()
    # same gradient formula; bf16 stored once (recompute) vs twice (forward, then x3)
    ref = OracleRef(host_logits(x.cpu()), t.cpu().numpy(), label_smoothing=0.1,
                    lse_square_scale=1e-3, reduction="mean")
    assert_grad_close(a.grad, ref.grad * 3.0, ref.mag * 3.0, zero_rows=ref.not_counted)


def test_determinism_bitwise():
    x = synth.make_logits(512, 32768, torch.bfloat16, 2.0, 71)
    t = synth.make_targets(512, 32768, 71, 20)
    outs = []
    for path in ("fused", "splitv", "fused", "splitv"):
        _announce(name="determinism", path=path)
        xd = x.to(DEV)
        r = forward_raw(xd, t.to(DEV), label_smoothing=0.1, lse_square_scale=1e-3,
                        z_loss=True, token_accuracy=True, argmax=True, counts=True,
                        flags=PATH_FLAGS[path])
        torch.cuda.synchronize()
        outs.append((xd.cpu(), [o.cpu() for o in r]))
    for a, b in ((0, 2), (1, 3)):
        assert torch.equal(outs[a][0].view(torch.int16), outs[b][0].view(torch.int16))
        for oa, ob in zip(outs[a][1], outs[b][1]):
            assert torch.equal(oa, ob)
    # fused vs split-V: identical integers, floats within the parity bar of each other
    assert torch.equal(outs[0][1][3], outs[1][1][3])
    assert torch.equal(outs[0][1][4], outs[1][1][4])
    assert abs(outs[0][1][0].item() - outs[1][1][0].item()) <= 1e-5 * abs(outs[0][1][0].item())


# ---------------------------------------------------------------------------
# Every fused row shape, with more rows than workgroups fit on the device at
# once (so the persistent row kernel claims rows dynamically), a ragged row
# tail, a partial last slot and many ignored rows; every element compared.
# ---------------------------------------------------------------------------

SHAPE_CASES = [
    # (dtype, V, rows, options): V picks the shape (the default layout / the
    # CE_F_SHAPE_ALT one where a row size has two); rows exceed the resident
    # grid, so persistent workgroups claim rows as they finish
    (torch.float32, 4001, 2600, dict()),                              # 256 x 4
    (torch.float32, 16001, 1100, dict(eps=0.1, lam=1e-3)),            # 256 x 16 / 1024 x 4
    (torch.float32, 65001, 300, dict(weight=True, eps=0.05)),         # 512 x 16 pair / 512 x 32
    (torch.float32, 129001, 300, dict(lam=1e-4)),                     # quarters / 1024 x 16 pair
    (torch.bfloat16, 16001, 2600, dict(softcap=20.0)),                # 256 x 8
    # 256 x 16 with rows claimed: the last block reduces 16 rows per thread per
    # round, so 4500 rows take a full round of 4096 and a ragged one
    (torch.bfloat16, 32001, 4500, dict(eps=0.05, lam=1e-4)),          # 256 x 16 / 1024 x 4
    (torch.bfloat16, 65001, 600, dict()),                             # 512 x 8 pair / 512 x 16
    (torch.bfloat16, 131001, 300, dict(weight=True, eps=0.1, softcap=30.0, lam=1e-4)),
    # the largest shapes with every per-element option (fewer rows: oracle time)
    (torch.float32, 130001, 40, dict(weight=True, eps=0.1, softcap=15.0)),    # quarters / pair
    (torch.bfloat16, 250001, 40, dict(eps=0.1, softcap=30.0, lam=1e-4)),      # quarters / pair
    (torch.bfloat16, 262001, 24, dict(weight=True, eps=0.2)),                 # quarters / pair
    # split rows: argmax and target in any part, a tie across parts, small
    # logits (|max| < 2: the argmax re-reads raw logits), no row tail
    (torch.float32, 128256, 64, dict(sigma=0.3, tie=1.5)),
    (torch.bfloat16, 262144, 48, dict(sigma=0.5, tie=4.0)),
]


@pytest.mark.parametrize("case", range(len(SHAPE_CASES)))
@pytest.mark.parametrize("reduction", ["mean", "none"])
@pytest.mark.parametrize("layout", ["fused", "fused_alt"])
def test_fused_shapes_many_rows(case, reduction, layout):
    dtype, V, rows, o = SHAPE_CASES[case]
    seed = 100 + case
    x = synth.make_logits(rows, V, dtype, o.get("sigma", 2.5), seed)
    t = synth.make_targets(rows, V, seed, rows * 3 // 10)
    if o.get("tie"):
        # equal maxima in the first and the last part of every other row (the
        # first one must win), the single maximum in the last part of the rest
        for r in range(rows):
            x[r, V - 5] = o["tie"]
            if r % 2 == 0:
                x[r, 7 + r] = o["tie"]
        t[1::4] = V - 3
    wt = None
    if o.get("weight"):
        wt = 0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(seed))
    stride = (V + 7) // 8 * 8  # 16-byte aligned rows: the vector path
    run_case(x, t, weight=wt, eps=o.get("eps", 0.0), lam=o.get("lam", 0.0),
             softcap=o.get("softcap"), reduction=reduction, path=layout, stride=stride,
             name=f"shape-{case}")


# Rows split over a group of workgroups (pairs, quarters) with fewer rows than
# the resident grid holds: the grid shrinks to rows x G workgroups, a
# multiple of G, and each group's part 0 still claims the next row (none).
SPLIT_CASES = [
    (torch.float32, 24001),    # 6000 vectors: 512 x 8 pair / 512 x 16 row kernel
    (torch.float32, 50001),    # 12500: 512 x 16 pair / 512 x 32 row kernel
    (torch.float32, 120001),   # 30000: quarter rows / 1024 x 16 pair
    (torch.bfloat16, 250001),  # 31250: quarter rows / 1024 x 16 pair
]


@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
@pytest.mark.parametrize("rows", [1, 2, 5])
@pytest.mark.parametrize("layout", ["fused", "fused_alt"])
def test_split_rows_few_rows(case, rows, layout):
    dtype, V = SPLIT_CASES[case]
    seed = 300 + 10 * case + rows
    x = synth.make_logits(rows, V, dtype, 2.0, seed)
    t = synth.make_targets(rows, V, seed, 1 if rows == 5 else 0)
    stride = (V + 7) // 8 * 8  # 16-byte aligned rows: the vector path
    run_case(x, t, eps=0.1, reduction="none", path=layout, stride=stride,
             name=f"split-{case}")


@pytest.mark.parametrize("alt", [False, True])
def test_persistent_claims_reset_between_calls(alt):
    """Row claims (persistent kernel) start from zero on every call and row
    pairs find only this call's partials: the same batch gives the same bits
    after calls of other sizes share the workspace."""
    V = 129001
    xa = synth.make_logits(600, V, torch.float32, 2.0, 91)
    ta = synth.make_targets(600, V, 91, 40)
    xb = synth.make_logits(290, V, torch.float32, 2.0, 92)
    tb = synth.make_targets(290, V, 92, 200)
    outs = []
    for x, t in ((xa, ta), (xb, tb), (xa, ta), (xb, tb), (xa, ta)):
        _announce(name="claims", rows=x.shape[0], V=V, alt=alt)
        xd = _padded(x, V + 7)
        flags = CE_F_SHAPE_ALT if alt else 0
        assert _plan(xd, None, 0.0, flags) == "fused"
        r = forward_raw(xd, t.to(DEV), reduction="sum", z_loss=True, token_accuracy=True,
                        argmax=True, counts=True, flags=flags)
        torch.cuda.synchronize()
        outs.append((xd.cpu(), [o.cpu() for o in r if o is not None]))
    for a, b in ((0, 2), (0, 4), (1, 3)):
        assert torch.equal(outs[a][0].view(torch.int32), outs[b][0].view(torch.int32))
        for oa, ob in zip(outs[a][1], outs[b][1]):
            assert torch.equal(oa, ob)


# ---------------------------------------------------------------------------
# The planner's own split-V path (no test hook): batches of fewer than 256
# rows with long rows, and rows longer than any fused shape holds. Chunks of
# up to 1024 vectors take the 256 x 4 stage 1, longer ones the 512 x 16 one.
# ---------------------------------------------------------------------------

AUTO_SPLITV = [
    # (dtype, V, rows, options); the comment gives the plan the library makes
    (torch.bfloat16, 262144, 8, dict(weight=True, eps=0.1, softcap=30.0, lam=1e-4)),  # S 32 x 1024
    (torch.bfloat16, 262144, 200, dict(weight=True, eps=0.1, softcap=30.0, lam=1e-4)),  # S 6 x 5462
    (torch.float32, 1048576, 64, dict(eps=0.05, lam=1e-4)),                           # S 32 x 8192
    (torch.float32, 262144, 300, dict(weight=True, eps=0.2)),                         # S 8 x 8192
    (torch.float32, 200003, 40, dict(softcap=15.0)),                                  # ragged tail
]


@pytest.mark.parametrize("case", range(len(AUTO_SPLITV)))
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_planner_splitv(case, reduction):
    dtype, V, rows, o = AUTO_SPLITV[case]
    seed = 500 + case
    x = synth.make_logits(rows, V, dtype, 2.0, seed)
    t = synth.make_targets(rows, V, seed, max(1, rows // 10))
    t[0] = V - 1  # a target in the last chunk (and the row tail)
    wt = None
    if o.get("weight"):
        wt = 0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(seed))
    stride = (V + 7) // 8 * 8
    xd = _padded(x, stride)
    assert _plan(xd, None if wt is None else wt.to(DEV), o.get("eps", 0.0), 0) == "splitv"
    del xd
    run_case(x, t, weight=wt, eps=o.get("eps", 0.0), lam=o.get("lam", 0.0),
             softcap=o.get("softcap"), reduction=reduction, path="auto", stride=stride,
             name=f"auto-splitv-{case}")


# ---------------------------------------------------------------------------
# Non-finite logits in counted rows: NaN makes the row's loss and gradient
# NaN and is the row's argmax (its first NaN), +inf makes the row NaN (its
# argmax stays the first +inf); with softcap, +inf saturates to the cap.
# ---------------------------------------------------------------------------

NAN_CASES = [
    # (dtype, V, rows, path, options)
    (torch.float32, 4099, 40, "fused", dict()),           # row kernel, exponentials kept
    (torch.float32, 4099, 40, "fused", dict(softcap=5.0)),
    (torch.bfloat16, 8195, 40, "fused", dict()),
    (torch.bfloat16, 8195, 40, "fused", dict(softcap=5.0, eps=0.1)),
    (torch.float32, 4099, 40, "splitv", dict()),
    (torch.bfloat16, 4099, 40, "splitv", dict(softcap=5.0)),
    (torch.float32, 4099, 40, "scalar", dict()),
    (torch.bfloat16, 4099, 40, "scalar", dict(softcap=5.0)),
    (torch.float32, 129001, 24, "fused", dict()),         # quarter rows
    (torch.float32, 129001, 24, "fused", dict(softcap=20.0, lam=1e-3)),
    (torch.bfloat16, 131001, 24, "fused", dict()),        # row pairs
    (torch.bfloat16, 131001, 24, "fused_alt", dict(eps=0.1)),
]


@pytest.mark.parametrize("case", range(len(NAN_CASES)))
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_nonfinite_logits_in_counted_rows(case, reduction):
    dtype, V, rows, path, o = NAN_CASES[case]
    seed = 700 + case
    x = synth.make_logits(rows, V, dtype, 2.0, seed)
    t = synth.make_targets(rows, V, seed, 3)
    g = torch.Generator().manual_seed(seed)
    cols = lambda k: torch.randperm(V, generator=g)[:k].tolist()  # noqa: E731
    for r in range(rows):
        kind = r % 6
        if kind == 0:
            x[r, cols(1)[0]] = float("nan")
        elif kind == 1:  # two NaNs and a large logit before them
            c = sorted(cols(3))
            x[r, c[0]] = 50.0
            x[r, c[1]] = float("nan")
            x[r, c[2]] = float("nan")
        elif kind == 2:
            x[r, cols(1)[0]] = float("inf")
        elif kind == 3:
            x[r, V - 1] = float("nan")  # in the row tail (V is not a multiple of a vector)
        elif kind == 4:
            x[r, cols(1)[0]] = float("-inf")
    stride = (V + 7) // 8 * 8 if path != "scalar" else V
    run_case(x, t, eps=o.get("eps", 0.0), lam=o.get("lam", 0.0), softcap=o.get("softcap"),
             reduction=reduction, path=path, stride=stride, name=f"nonfinite-{case}")


# ---------------------------------------------------------------------------
# A split row's exchange that gives up is loud: forced from the host
# (CE_F_EXCHANGE_ONE_POLL: one poll before giving up), every kernel still
# ends normally, CE_F_CHECK_TARGETS reports CE_E_EXCHANGE, the reduced
# outputs are NaN, and every value is either NaN or the oracle's.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,V,rows,layout", [(torch.float32, 129001, 300, "fused"),
                                                 (torch.bfloat16, 131001, 300, "fused"),
                                                 (torch.float32, 129001, 300, "fused_alt")])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_exchange_timeout_is_loud(dtype, V, rows, layout, reduction):
    seed = 900 + V % 97
    x = synth.make_logits(rows, V, dtype, 2.0, seed)
    t = synth.make_targets(rows, V, seed, rows // 10)
    stride = (V + 7) // 8 * 8
    xd = _padded(x, stride)
    td = t.to(DEV)
    flags = PATH_FLAGS[layout] | CE_F_EXCHANGE_ONE_POLL | _lib.CE_F_GRAD | _lib.CE_F_CHECK_TARGETS
    _announce(name="exchange-timeout", rows=rows, V=V, dtype=dtype, reduction=reduction,
              layout=layout, plan=_plan(xd, None, 0.0, flags))
    assert _plan(xd, None, 0.0, flags) == "fused"
    dt = _lib.dtype_code(dtype)
    shape = (rows,) if reduction == "none" else ()
    loss = torch.empty(shape, device=DEV)
    acc = torch.empty(shape, device=DEV)
    arg = torch.empty((rows,), device=DEV, dtype=torch.int64)
    counts = torch.empty((2,), device=DEV, dtype=torch.int64)
    wsb = _lib.ce_workspace_bytes(rows, V, dt, flags)
    ws = torch.zeros((wsb,), device=DEV, dtype=torch.uint8)
    s = torch.cuda.current_stream().cuda_stream
    st = _lib.ce_forward(xd.data_ptr(), dt, rows, V, stride, td.data_ptr(), 0, -100, 0.0, 0.0,
                         0.0, _lib.REDUCTION_CODES[reduction], flags, loss.data_ptr(), 0,
                         acc.data_ptr(), arg.data_ptr(), counts.data_ptr(), 0, ws.data_ptr(),
                         wsb, s)
    torch.cuda.synchronize()
    assert st == _lib.CE_E_EXCHANGE, _lib.ce_status_string(st)
    ref = OracleRef(host_logits(x), t.numpy(), reduction=reduction)
    if reduction == "none":
        lg = loss.cpu().double().numpy()
        ok = ~np.isnan(lg)
        assert not ok.all(), "no row carries the failure"
        assert_loss_close(lg[ok], np.asarray(ref.loss)[ok], "per-row loss (rows not poisoned)")
    else:
        assert math.isnan(loss.item()) and math.isnan(acc.item())
    am = arg.cpu().numpy()
    assert np.all((am == -1) | (am == ref.argmax))
    g = x_cpu_grad = xd.detach().float().cpu().double().numpy()
    nan = np.isnan(g)
    assert nan.any() and not nan[ref.not_counted].any()
    # every value that is not NaN is the oracle's
    filled = torch.from_numpy(np.where(nan, ref.grad, g)).to(dtype)
    assert_grad_close(filled, ref.grad, ref.mag, zero_rows=ref.not_counted,
                      what="gradient outside the poisoned parts")
    del x_cpu_grad
    # the next call on the same workspace, without the hook, is clean
    xd2 = _padded(x, stride)
    flags2 = flags & ~CE_F_EXCHANGE_ONE_POLL
    st = _lib.ce_forward(xd2.data_ptr(), dt, rows, V, stride, td.data_ptr(), 0, -100, 0.0, 0.0,
                         0.0, _lib.REDUCTION_CODES[reduction], flags2, loss.data_ptr(), 0,
                         acc.data_ptr(), arg.data_ptr(), counts.data_ptr(), 0, ws.data_ptr(),
                         wsb, s)
    torch.cuda.synchronize()
    assert st == _lib.CE_OK, _lib.ce_status_string(st)
    assert_loss_close(loss.cpu().numpy(), ref.loss, "loss after a clean call")
    np.testing.assert_array_equal(arg.cpu().numpy(), ref.argmax)
    assert_grad_close(xd2, ref.grad, ref.mag, zero_rows=ref.not_counted)


# ---------------------------------------------------------------------------
# Full-size workloads in the benchmark's launch configuration, against the
# oracle on every row: loss, z-loss, token accuracy, argmax and counts of
# the whole batch, and every row's gradient (a seeded sample of rows at
# 16384 x 262144, where the float64 gradient of every row would take the
# host minutes).
# ---------------------------------------------------------------------------

def _sample_rows(rows, k, seed, extra=()):
    g = np.random.default_rng(seed)
    s = set(g.choice(rows, size=min(k, rows), replace=False).tolist())
    s.update([0, rows - 1])
    s.update(int(e) for e in extra)
    return np.array(sorted(s))


def _full_workload(name, grad_sample=None, grad=True):
    """grad=False: the forward without the gradient (it also saves the per-row
    statistics), and the gradient recomputed from those is what is compared."""
    w = synth.WORKLOADS[name] if isinstance(name, str) else name
    for red in w.reductions:
        _announce(name=w.name, rows=w.rows, V=w.V, dtype=w.dtype, reduction=red, grad=grad)
        inp = synth.make_inputs(w, DEV)
        x = inp.logits
        xh = host_logits(x)  # every row, before the forward overwrites them
        t_host = inp.target.cpu().numpy()
        wh = None if inp.weight is None else inp.weight.cpu().numpy()
        opts = dict(weight=wh, label_smoothing=w.label_smoothing,
                    lse_square_scale=w.lse_square_scale, softcap=w.softcap or None)
        stats = None if grad else torch.empty((w.rows, 2), device=DEV, dtype=torch.float32)
        loss, z, acc, arg, counts = forward_raw(
            x, inp.target, inp.weight, -100, w.label_smoothing, w.lse_square_scale,
            w.softcap or None, red, grad=grad, z_loss=True, token_accuracy=True, argmax=True,
            counts=True, row_stats=stats)
        gsrc = x
        if not grad:
            go = (torch.ones(w.rows, device=DEV) if red == "none"
                  else torch.tensor(1.0, device=DEV))
            gsrc = backward_recompute(x, inp.target, inp.weight, -100, w.label_smoothing,
                                      w.lse_square_scale, w.softcap or None, red, stats, go)
        torch.cuda.synchronize()
        print(f"  gpu done; oracle over {w.rows} rows", flush=True)
        o, summ = oracle_rows(xh, t_host, reduction=red, **opts)
        want_loss, want_z, want_acc, n_correct = reduce_rows(
            o["ce"], o["zeta"], o["correct"], summ.counted, summ.n, summ.D, red)
        np.testing.assert_array_equal(arg.cpu().numpy(), o["argmax"])
        c = counts.cpu().numpy()
        assert int(c[0]) == summ.n and int(c[1]) == n_correct
        if red == "none":
            assert_loss_close(loss.cpu().numpy(), want_loss, "per-row loss")
            assert_loss_close(z.cpu().numpy(), want_z, "per-row z_loss")
            np.testing.assert_array_equal(acc.cpu().numpy(), want_acc.astype(np.float32))
        else:
            assert_loss_close(np.array(loss.item()), np.array(want_loss), "loss")
            assert_loss_close(np.array(z.item()), np.array(want_z), "z_loss")
            assert_acc_exact(acc.item(), n_correct, summ.n)
        sel = (np.arange(w.rows) if grad_sample is None else
               _sample_rows(w.rows, grad_sample, w.seed, inp.spike_rows))
        print(f"  scalars and argmax match; gradients of {sel.size} rows", flush=True)
        for a in range(0, sel.size, 512):
            rr = sel[a:a + 512]
            og, _ = oracle_rows(xh, t_host, reduction=red, want_grad=True, rows=rr, **opts)
            assert_grad_close(gsrc[torch.from_numpy(rr).to(DEV)], og["grad"], og["mag"],
                              zero_rows=~summ.counted[rr], what=f"{w.name} grad rows {rr[0]}..")
        del inp, x, xh, gsrc


def test_full_c2_bf16_accuracy_argmax():
    _full_workload("ce_4096x32768_bf16")


def test_full_c3_f32_large_vocab():
    _full_workload("ce_1023x128256_f32")


def test_full_c4_bf16_all_options():
    _full_workload("ce_4096x131072_bf16_opts")


def test_full_c5_bf16_huge():
    _full_workload("ce_16384x262144_bf16", grad_sample=512)


def test_full_c3_nograd_streamed():
    """The headline batch without the gradient (each row streamed through one
    workgroup): every scalar and argmax, and every row's gradient recomputed
    from the saved row statistics."""
    _full_workload("ce_1023x128256_f32", grad=False)


def test_full_c4_nograd_streamed():
    _full_workload("ce_4096x131072_bf16_opts", grad=False, grad_sample=512)


def test_quarter_rows_many_rows_per_group_f32():
    """fp32 rows of 16400 vectors (quarter rows) in a batch of 4200, about 33
    rows per group of four resident workgroups (the headline batch has 8):
    every row's scalars and argmax, and a sample of gradients, against the
    oracle."""
    base = synth.WORKLOADS["ce_1023x128256_f32"]
    w = dataclasses.replace(base, name="ce_4200x65600_f32", rows=4200, V=65600,
                            reductions=("mean",))
    _full_workload(w, grad_sample=256)
