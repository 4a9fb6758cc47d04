"""GPU checks of ce_forward_noalloc (the forward on the library's static
device scratch) against ce_forward with a workspace of its own.

Each case makes two calls in a row through the C ABI, the second on a
smaller problem, so the second runs on the scratch the first left behind.
Both entry points share their kernels: every output (loss, z-loss, token
accuracy, argmax, counts, row statistics, the gradient) must be the same
bits, and the no-alloc results must also meet the oracle's tolerances.
"""

import numpy as np
import pytest
import torch

import synth
from parity import OracleRef, assert_grad_close, assert_loss_close, host_logits
from softmax_cross_entropy_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (dtype, rows, V, options); the second call of a pair is smaller than the first
PAIRS = [
    # rows split over groups of workgroups (exchange slots in the scratch),
    # then one workgroup per row
    [(torch.float32, 96, 70000, dict(weight=True, eps=0.1, lam=1e-4, red="mean")),
     (torch.bfloat16, 50, 4096, dict(red="sum"))],
    # the split-V path (partials in the scratch), then a smaller split-V call
    [(torch.bfloat16, 160, 50000, dict(path="splitv", softcap=30.0, red="none")),
     (torch.float32, 37, 3003, dict(path="splitv", weight=True, eps=0.2, red="mean"))],
    # the benchmark's bf16 shape class, then a tiny batch with ignored rows
    [(torch.bfloat16, 512, 32768, dict(red="mean")),
     (torch.float32, 8, 1000, dict(red="mean", ignore_all_but=2))],
]


def _announce(**kw):
    print("CASE " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _call(entry, x, t, w, o, ws=None):
    """One forward (+ gradient) through `entry`; returns every output on the host."""
    rows, V = x.shape
    red = o.get("red", "mean")
    flags = _lib.CE_F_GRAD | {"splitv": _lib.CE_F_FORCE_SPLITV}.get(o.get("path"), 0)
    shape = (rows,) if red == "none" else ()
    loss, z, acc = (torch.full(shape, 7.0, device=DEV) for _ in range(3))
    arg = torch.full((rows,), -7, dtype=torch.int64, device=DEV)
    cnt = torch.full((2,), -7, dtype=torch.int64, device=DEV)
    stats = torch.full((rows, 2), 7.0, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), _lib.dtype_code(x.dtype), rows, V, x.stride(0), t.data_ptr(),
            0 if w is None else w.data_ptr(), -100, o.get("eps", 0.0), o.get("lam", 0.0),
            o.get("softcap", 0.0), _lib.REDUCTION_CODES[red], flags, loss.data_ptr(),
            z.data_ptr(), acc.data_ptr(), arg.data_ptr(), cnt.data_ptr(), stats.data_ptr())
    if entry == "noalloc":
        st = _lib.ce_forward_noalloc(*args, s)
    else:
        st = _lib.ce_forward(*args, ws.data_ptr(), ws.numel(), s)
    assert st == _lib.CE_OK, f"{entry}: {_lib.ce_status_string(st)}"
    torch.cuda.synchronize()
    return dict(loss=loss.cpu(), z=z.cpu(), acc=acc.cpu(), arg=arg.cpu(), cnt=cnt.cpu(),
                stats=stats.cpu(), grad=x.cpu())


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32) \
        if t.dtype == torch.float32 else t


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_forward_twice(pair):
    for k, (dtype, rows, V, o) in enumerate(PAIRS[pair]):
        seed = 3100 + 10 * pair + k
        x = synth.make_logits(rows, V, dtype, 2.0, seed)
        t = synth.make_targets(rows, V, seed, rows // 10)
        if o.get("ignore_all_but"):
            t[o["ignore_all_but"]:] = -100
        wt = (0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(seed))
              if o.get("weight") else None)
        _announce(name="noalloc", pair=pair, call=k, rows=rows, V=V, dtype=dtype, options=o)
        xd_a, xd_b = x.to(DEV), x.to(DEV)
        td = t.to(DEV)
        wd = None if wt is None else wt.to(DEV)
        flags = _lib.CE_F_GRAD | {"splitv": _lib.CE_F_FORCE_SPLITV}.get(o.get("path"), 0)
        wsb = _lib.ce_workspace_bytes(rows, V, _lib.dtype_code(dtype), flags)
        assert wsb <= _lib.CE_FORWARD_NOALLOC_MAX_BYTES
        ws = torch.zeros((wsb,), dtype=torch.uint8, device=DEV)
        want = _call("forward", xd_a, td, wd, o, ws)
        got = _call("noalloc", xd_b, td, wd, o)
        for key in want:
            assert torch.equal(_bits(got[key]), _bits(want[key])), f"call {k}: {key} differs"
        # and the oracle's tolerances, as for ce_forward
        red = o.get("red", "mean")
        ref = OracleRef(host_logits(x), t.numpy(), weight=None if wt is None else wt.numpy(),
                        label_smoothing=o.get("eps", 0.0), lse_square_scale=o.get("lam", 0.0),
                        softcap=o.get("softcap"), reduction=red)
        assert_loss_close(got["loss"].numpy(), ref.loss, "loss")
        assert_loss_close(got["z"].numpy(), ref.z_loss, "z_loss")
        np.testing.assert_array_equal(got["arg"].numpy(), ref.argmax)
        assert int(got["cnt"][0]) == ref.summ.n and int(got["cnt"][1]) == ref.n_correct
        assert_grad_close(xd_b, ref.grad, ref.mag, zero_rows=ref.not_counted,
                          what="no-alloc gradient")
