"""GPU parity of the vocabulary-parallel cross-entropy (ce_shard_partials,
ce_shard_finish) against the float64 oracle on the full rows.

One device plays every shard: the (rows, V_total) batch is split into G
column slices, stage 1 runs on each slice, the G partial arrays are placed
side by side (what the all-gather of a multi-device run delivers), and stage
2 runs on each slice. Every shard must return the same outputs, equal to the
oracle's over all V_total classes, and together the slices must hold the
full gradient. Tolerances are those of tests/parity.py.
"""

import numpy as np
import pytest
import torch

import synth
from parity import OracleRef, assert_acc_exact, assert_grad_close, assert_loss_close, host_logits
from softmax_cross_entropy_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # (dtype, rows, V_total, shards, options)
    (torch.float32, 1023, 128256, 8, dict()),                  # the headline batch, 8 x 16032
    (torch.bfloat16, 64, 131072, 4, dict(weight=True, eps=0.1, softcap=30.0, lam=1e-4)),
    (torch.float32, 37, 3003, 3, dict(weight=True, eps=0.2, softcap=4.0, lam=1e-2)),  # unaligned
    (torch.bfloat16, 40, 20008, 1, dict(weight=True, eps=0.1)),  # one shard: the whole row
    (torch.bfloat16, 50, 24000, 3, dict(tie=True)),            # ties and NaN across shards
]


def _announce(**kw):
    print("CASE " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_shards_match_oracle(case, reduction):
    dtype, rows, V, G, o = CASES[case]
    seed = 1200 + case
    x = synth.make_logits(rows, V, dtype, 2.0, seed)
    t = synth.make_targets(rows, V, seed, rows // 10)
    t[0] = V - 1
    if o.get("tie"):
        # equal maxima in two different shards (the lower index must win), and
        # a NaN in the last shard of a row (it is that row's argmax)
        for r in range(0, rows, 2):
            x[r, 5] = 9.0
            x[r, V - 7] = 9.0
        x[3, V - 2] = float("nan")
    wt = (0.5 + 1.5 * torch.rand(V, generator=torch.Generator().manual_seed(seed))
          if o.get("weight") else None)
    eps, lam, cap = o.get("eps", 0.0), o.get("lam", 0.0), o.get("softcap")
    xd = x.to(DEV)
    td = t.to(DEV)
    wd = None if wt is None else wt.to(DEV)
    dt = _lib.dtype_code(dtype)
    eb = x.element_size()
    bounds = [V * g // G for g in range(G + 1)]
    _announce(name="shards", rows=rows, V=V, shards=G, dtype=dtype, reduction=reduction,
              options=o, slices=bounds[:3])
    s = torch.cuda.current_stream().cuda_stream
    P = lambda a: 0 if a is None else a.data_ptr()  # noqa: E731
    parts = torch.zeros((G, rows, 32), dtype=torch.uint8, device=DEV)
    for g in range(G):
        off, Vl = bounds[g], bounds[g + 1] - bounds[g]
        st = _lib.ce_shard_partials(xd.data_ptr() + off * eb, dt, rows, Vl, V, off, V, P(td),
                                    P(wd), -100, eps, cap or 0.0, parts[g].data_ptr(), s)
        assert st == 0, _lib.ce_status_string(st)
    shape = (rows,) if reduction == "none" else ()
    outs = []
    wsb = _lib.ce_shard_workspace_bytes(rows)
    for g in range(G):
        off, Vl = bounds[g], bounds[g + 1] - bounds[g]
        o_ = [torch.empty(shape, device=DEV) for _ in range(3)]
        arg = torch.empty((rows,), dtype=torch.int64, device=DEV)
        cnt = torch.empty((2,), dtype=torch.int64, device=DEV)
        ws = torch.zeros((wsb,), dtype=torch.uint8, device=DEV)
        st = _lib.ce_shard_finish(xd.data_ptr() + off * eb, dt, rows, Vl, V, off, V, P(td), P(wd),
                                  -100, eps, lam, cap or 0.0, _lib.REDUCTION_CODES[reduction], 0,
                                  parts.data_ptr(), G, o_[0].data_ptr(), o_[1].data_ptr(),
                                  o_[2].data_ptr(), arg.data_ptr(), cnt.data_ptr(),
                                  ws.data_ptr(), wsb, s)
        assert st == 0, _lib.ce_status_string(st)
        outs.append((o_, arg, cnt))
    torch.cuda.synchronize()
    ref = OracleRef(host_logits(x), t.numpy(), weight=None if wt is None else wt.numpy(),
                    label_smoothing=eps, lse_square_scale=lam, softcap=cap, reduction=reduction)
    (loss, z, acc), arg, cnt = outs[0]
    for (o2, a2, c2) in outs[1:]:  # every shard the same bits
        for u, v in zip((loss, z, acc), o2):
            assert torch.equal(u.view(torch.int32), v.view(torch.int32))
        assert torch.equal(arg, a2) and torch.equal(cnt, c2)
    assert_loss_close(loss.cpu().numpy(), ref.loss, "loss")
    assert_loss_close(z.cpu().numpy(), ref.z_loss, "z_loss")
    np.testing.assert_array_equal(arg.cpu().numpy(), ref.argmax)
    c = cnt.cpu().numpy()
    assert int(c[0]) == ref.summ.n and int(c[1]) == ref.n_correct
    if reduction == "none":
        np.testing.assert_array_equal(acc.cpu().numpy(), ref.acc.astype(np.float32))
    else:
        assert_acc_exact(acc.item(), ref.n_correct, ref.summ.n)
    assert_grad_close(xd, ref.grad, ref.mag, zero_rows=ref.not_counted, what="sharded gradient")
