"""Benchmark of the fused softmax cross-entropy forward + gradient on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode MODE]

A step is one pass of the whole hot path over one batch of synthetic logits
already resident in HBM: ce_forward (loss + gradient written over the
logits) followed by ce_backward with grad_output = 1 (the training call
pattern). Every step gets its own pristine copy of the batch (prepared
before the timed region), so no step reads a gradient left by another.
--mode nograd times the forward without the gradient (an evaluation pass);
--mode recompute keeps the logits and times the gradient recomputed from
them (ce_backward_recompute) after that forward.

The default workload is 1023 rows x V = 128256 fp32 logits, reduction
"sum" (the tt-mlir PR #9324 page's before/after shape). Prints one JSON
line with rows/s, the roofline of the fused kernel (achieved HBM GB/s from
algorithmic bytes over its event-timed duration) and the float64 oracle
timed on the host cores as a CPU baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "ce_1023x128256_f32"
DEFAULT_REDUCTION = {"ce_1023x128256_f32": "sum"}
PROFILES = os.path.join(ROOT, "profiles")


def source_hash() -> str:
    """Hash of the HIP sources: counter-based traffic figures are valid only
    for the kernels they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "softmax_cross_entropy_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, reduction: str, n_counted: int, mode: str = "fused") -> int:
    """Bytes the method itself must move in the timed kernel: each counted row
    read once, every row's gradient written once (not in the no-gradient
    forward), targets, class weights and the outputs; the recomputing
    backward also reads the per-row statistics."""
    e = w.elem_bytes
    b = n_counted * w.V * e + w.rows * 8
    if mode != "nograd":
        b += w.rows * w.V * e
    if mode == "recompute":
        b += w.rows * 8
        return b
    if w.weights:
        b += w.V * 4
    n_out = 1 + (1 if w.want_z_loss else 0) + (1 if w.want_accuracy else 0)
    b += (w.rows * 4 if reduction == "none" else 4) * n_out
    if w.want_argmax:
        b += w.rows * 8
    return b


def traffic_from_profiles(workload: str, kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on different kernel sources."""
    path = os.path.join(PROFILES, f"{kernel_key}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_per_kernel(csv_path: str, counter: str):
    """Per-dispatch values (KiB) of one rocprofv3 --pmc counter, by kernel name."""
    import csv
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def write_traffic(workload: str, fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes per launch of the fused kernel from two rocprofv3 --pmc runs of
    this benchmark (FETCH_SIZE, then WRITE_SIZE). Each counter is scaled by
    what it reads for the runtime's copy kernel moving the logits buffer (a
    known size: every step's pristine copy of the batch), and the result is
    stored under profiles/ with the hash of the kernel sources it was taken on."""
    import synth
    w = synth.WORKLOADS[workload]
    nbytes = w.rows * w.V * w.elem_bytes
    rec = {"workload": workload, "source_hash": source_hash(), "copy_bytes": nbytes}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = _pmc_per_kernel(path, counter)
        copies = [v for k, vs in per.items() if "copyBuffer" in k for v in vs]
        big = [v for v in copies if v >= 0.9 * max(copies)]
        factor = nbytes / (sum(big) / len(big) * 1024.0)
        kern = {k: vs for k, vs in per.items() if "rows_kernel" in k or "wide_kernel" in k}
        if len(kern) != 1:
            raise SystemExit(f"expected one fused kernel in {path}, found {list(kern)}")
        name, vs = next(iter(kern.items()))
        raw = sum(vs) / len(vs) * 1024.0
        rec[counter] = {"kernel": name, "dispatches": len(vs), "raw_bytes": raw,
                        "copy_dispatches": len(big), "copy_factor": factor,
                        "bytes": raw * factor}
        total += raw * factor
    rec["hbm_bytes_per_launch"] = total
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"ce_fused_{workload}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return rec


def sweep(steps: int, warmup: int, extra_flags: int = 0) -> None:
    """Context numbers: the Liger CE profile's benchmark sweep shape (B=8, T=512
    rows, bf16, V from 4096 to 131072, mean) for this library's fused forward +
    gradient + backward step, next to PyTorch eager F.cross_entropy forward +
    backward on the same GPU and batch. One JSON line per V."""
    import torch
    import torch.nn.functional as F
    import synth
    from softmax_cross_entropy_amd import _lib
    from softmax_cross_entropy_amd.functional import _workspace

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = 8 * 512
    for V in (4096, 8192, 16384, 32768, 65536, 131072):
        x0 = synth.make_logits(rows, V, torch.bfloat16, 1.0, 200 + V, dev)
        t = synth.make_targets(rows, V, 200 + V, rows // 20).to(dev)
        nb = steps + warmup
        bufs = [x0.clone() for _ in range(nb)]
        loss = torch.empty((), device=dev, dtype=torch.float32)
        go = torch.ones((), device=dev, dtype=torch.float32)
        dt = _lib.CE_BF16
        wsb = _lib.ce_workspace_bytes(rows, V, dt, _lib.CE_F_GRAD | extra_flags)
        ws = _workspace(dev, wsb)
        s = stream.cuda_stream

        def ours(b):
            _lib.check(_lib.ce_forward(b.data_ptr(), dt, rows, V, V, t.data_ptr(), 0, -100, 0.0,
                                       0.0, 0.0, _lib.CE_RED_MEAN, _lib.CE_F_GRAD | extra_flags,
                                       loss.data_ptr(), 0, 0, 0, 0, 0, ws.data_ptr(), wsb, s),
                       "ce_forward")
            _lib.check(_lib.ce_backward(b.data_ptr(), dt, rows, V, V, go.data_ptr(), 0, s),
                       "ce_backward")

        def eager(b):
            xb = b.requires_grad_(True)
            F.cross_entropy(xb, t, ignore_index=-100).backward()
            xb.grad = None
            xb.requires_grad_(False)

        res = {}
        for name, fn in (("this_library", ours), ("torch_eager", eager)):
            for i in range(warmup):
                fn(bufs[i])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                fn(bufs[warmup + i])
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / steps
            bufs = [x0.clone() for _ in range(nb)]
        nbytes = 2 * rows * V * 2
        print(json.dumps({"sweep": "Liger CE profile benchmark shape (B=8, T=512, bf16, mean)",
                          "V": V, "rows": rows,
                          "ms_per_step": res,
                          "speedup_vs_torch_eager": res["torch_eager"] / res["this_library"],
                          "GBps_1R1W": {k: nbytes / (v * 1e-3) / 1e9 for k, v in res.items()}}),
              flush=True)
        del bufs, x0


def linear_bench(steps: int, warmup: int, rows: int = 4096, H: int = 4096, V: int = 128256,
                 chunk_rows: int = 0) -> None:
    """The linear layer fused with the cross-entropy at a language-model head
    shape (B=8, T=512 rows, hidden 4096, V = 128256, bf16), mean reduction:
    one step = ce_linear_forward with both gradients (grad_output = 1, so the
    backward's scaling exits at once), against PyTorch eager (bf16 matmul,
    fp32 cross-entropy, autograd) on the same GPU. Matrix-core roofline:
    6 rows V H flops per step (three products) against the bf16 dense peak."""
    import torch
    import torch.nn.functional as F
    import synth
    from softmax_cross_entropy_amd import linear_forward_raw

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    x = (torch.randn(rows, H, device=dev, generator=g) * 0.5).to(torch.bfloat16)
    w = (torch.randn(V, H, device=dev, generator=g) * (2.0 / H ** 0.5)).to(torch.bfloat16)
    t = synth.make_targets(rows, V, 7, rows // 20).to(dev)

    def ours():
        linear_forward_raw(x, w, t, reduction="mean", grad=True, chunk_rows=chunk_rows)

    def eager():
        xe = x.detach().requires_grad_(True)
        we = w.detach().requires_grad_(True)
        loss = F.cross_entropy((xe @ we.t()).float(), t, ignore_index=-100)
        loss.backward()

    res = {}
    for name, fn in (("this_library", ours), ("torch_eager", eager)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    flops = 6.0 * rows * V * H
    tf = flops / (res["this_library"] * 1e-3) / 1e12
    print(json.dumps({
        "linear": "linear layer fused with the cross-entropy (hidden @ weight^T, CE, both "
                  "gradients), mean, bf16 inputs",
        "config": {"rows": rows, "H": H, "V": V, "chunk_rows": chunk_rows or "default"},
        "ms_per_step": res,
        "speedup_vs_torch_eager": res["torch_eager"] / res["this_library"],
        "roofline": {"bound": "mfma", "achieved": tf, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tf / 2500.0, "flops_per_step": flops}}), flush=True)


def cpu_baseline(x_host, t_host, weight_host, w, reduction, budget_s=12.0):
    """Time the float64 oracle, as it is, on a bounded sample of the rows."""
    import numpy as np
    from oracle import ce_forward as oracle_forward

    rows_per_call = 64
    done_rows = 0
    t0 = time.perf_counter()
    c0 = resource.getrusage(resource.RUSAGE_SELF)
    calls = 0
    while True:
        a = (calls * rows_per_call) % max(1, x_host.shape[0] - rows_per_call)
        oracle_forward(x_host[a:a + rows_per_call], t_host[a:a + rows_per_call],
                       weight=weight_host, label_smoothing=w.label_smoothing,
                       lse_square_scale=w.lse_square_scale, softcap=w.softcap or None,
                       reduction=reduction)
        calls += 1
        done_rows += rows_per_call
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    c1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (c1.ru_utime - c0.ru_utime) + (c1.ru_stime - c0.ru_stime)
    cores = max(1, int(round(cpu / wall)))
    del np
    return {"value": done_rows / wall, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{calls} oracle calls of {rows_per_call} rows of the {w.name} batch "
                      f"({done_rows} rows, {wall:.1f} s wall, {cpu:.1f} s CPU)"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--reduction", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--mode", choices=("fused", "nograd", "recompute"), default="fused",
                    help="fused: forward + gradient in place, then the scaling backward "
                         "(default); nograd: forward without the gradient (logits only "
                         "read); recompute: forward without the gradient, then the gradient "
                         "recomputed from the kept logits into another buffer (roofline of "
                         "the recomputing kernel)")
    ap.add_argument("--path", choices=("auto", "fused", "splitv", "scalar"), default="auto",
                    help="force a kernel path (default: the library's choice)")
    ap.add_argument("--alt-shape", action="store_true",
                    help="the other fused layout for rows of 2 K to 32 K 16-byte vectors "
                         "(test hook, for comparing layouts)")
    ap.add_argument("--linear", action="store_true",
                    help="the linear layer fused with the cross-entropy at 4096 x 4096 hidden, "
                         "V = 128256 (JSON line with its matrix-core roofline), then exit")
    ap.add_argument("--chunk-rows", type=int, default=0,
                    help="--linear: rows per chunk (0: the library's default)")
    ap.add_argument("--sweep", action="store_true",
                    help="context sweep over V at the Liger benchmark shape, this library "
                         "against PyTorch eager F.cross_entropy (JSON line per V), then exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the fused kernel's HBM traffic from two rocprofv3 --pmc "
                         "counter_collection.csv files of this benchmark, then exit")
    a = ap.parse_args(argv)
    if a.traffic:
        write_traffic(a.workload, *a.traffic)
        return 0

    if a.linear:
        linear_bench(a.steps, a.warmup, chunk_rows=a.chunk_rows)
        return 0

    if a.sweep:
        from softmax_cross_entropy_amd import _lib
        sweep(a.steps, a.warmup, _lib.CE_F_SHAPE_ALT if a.alt_shape else 0)
        return 0

    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the path shards "
              "by rows, with no communication between GPUs on the hot path).", file=sys.stderr)
        return 2

    import torch
    import synth
    from softmax_cross_entropy_amd import _lib
    from softmax_cross_entropy_amd.functional import _workspace

    w = synth.WORKLOADS[a.workload]
    red = a.reduction or DEFAULT_REDUCTION.get(w.name, w.reductions[0])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    inp = synth.make_inputs(w, dev)
    t_host = inp.target.cpu().numpy()
    n_counted = int(((t_host != -100) & (t_host >= 0) & (t_host < w.V)).sum())
    nbuf = a.warmup + a.steps
    bufs = [inp.logits.clone() for _ in range(nbuf)]
    sample_host = None
    if not a.no_cpu_baseline:
        x = inp.logits[:256].detach().cpu()
        sample_host = (x.view(torch.int16).numpy().view("uint16") if x.dtype == torch.bfloat16
                       else x.numpy(), t_host[:256])
    dt = _lib.dtype_code(w.dtype)
    flags = _lib.CE_F_GRAD if a.mode == "fused" else 0
    flags |= {"auto": 0, "fused": _lib.CE_F_FORCE_FUSED, "splitv": _lib.CE_F_FORCE_SPLITV,
              "scalar": _lib.CE_F_FORCE_SCALAR}[a.path]
    if a.alt_shape:
        flags |= _lib.CE_F_SHAPE_ALT
    rows, V = w.rows, w.V
    f32 = dict(device=dev, dtype=torch.float32)
    loss = torch.empty((rows,) if red == "none" else (), **f32)
    z_loss = torch.empty_like(loss) if w.want_z_loss else None
    acc = torch.empty_like(loss) if w.want_accuracy else None
    arg = torch.empty((rows,), device=dev, dtype=torch.int64) if w.want_argmax else None
    go = torch.ones((), **f32)
    stats = torch.empty((rows, 2), **f32) if a.mode == "recompute" else None
    gbuf = torch.empty_like(inp.logits) if a.mode == "recompute" else None
    ws_bytes = _lib.ce_workspace_bytes(rows, V, dt, flags)
    ws = _workspace(dev, ws_bytes)
    P = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
    tgt, wt = P(inp.target), P(inp.weight)
    s = stream.cuda_stream
    path = _lib.PATH_NAMES[_lib.ce_plan_path(P(bufs[0]), dt, rows, V, bufs[0].stride(0), wt,
                                             w.label_smoothing, flags)]
    red_code = _lib.REDUCTION_CODES[red]

    def fwd(buf):
        st = _lib.ce_forward(P(buf), dt, rows, V, buf.stride(0), tgt, wt, -100,
                             w.label_smoothing, w.lse_square_scale, w.softcap, red_code, flags,
                             P(loss), P(z_loss), P(acc), P(arg), 0, P(stats), P(ws), ws_bytes, s)
        if st:
            raise _lib.CEError(st, "ce_forward")

    def bwd(buf):
        if a.mode == "fused":
            st = _lib.ce_backward(P(buf), dt, rows, V, buf.stride(0), P(go), 0, s)
        elif a.mode == "recompute":
            st = _lib.ce_backward_recompute(P(buf), dt, rows, V, buf.stride(0), tgt, wt, -100,
                                            w.label_smoothing, w.lse_square_scale, w.softcap,
                                            red_code, P(stats), P(go), 0, P(gbuf),
                                            gbuf.stride(0), P(ws), ws_bytes, s)
        else:
            st = 0
        if st:
            raise _lib.CEError(st, "backward")

    # The timed kernel: the fused forward, or the recomputing backward.
    timed_first = a.mode != "recompute"
    for i in range(a.warmup):
        fwd(bufs[i])
        bwd(bufs[i])
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(a.steps):
        b = bufs[a.warmup + i]
        if timed_first:
            ev[i][0].record(stream)
            fwd(b)
            ev[i][1].record(stream)
            bwd(b)
        else:
            fwd(b)
            ev[i][0].record(stream)
            bwd(b)
            ev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    fwd_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    kernel_ms = sum(fwd_ms) / len(fwd_ms)
    ms_per_step = total_ms / a.steps
    del bufs

    # copy ceiling of the same size (read + write), for context
    src = inp.logits
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * src.element_size() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del dst

    alg = algorithmic_bytes(w, red, n_counted, a.mode)
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    kernel_key = "ce_fused" if path == "fused" else f"ce_{path}"
    traffic = traffic_from_profiles(w.name, kernel_key) if a.mode == "fused" else None
    out = {
        "metric": "fused CE fwd+grad rows/s and achieved HBM GB/s (% of peak), V=128256",
        "value": rows * a.steps / (total_ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == torch.float32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": a.mode, "rows": rows, "V": V,
                   "reduction": red, "path": path,
                   "layout": "alternative" if a.alt_shape else "default",
                   "label_smoothing": w.label_smoothing, "softcap": w.softcap,
                   "lse_square_scale": w.lse_square_scale, "class_weights": w.weights,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel_ms": kernel_ms, "algorithmic_bytes": alg},
        "copy_ceiling_GBps": copy_gbps,
    }
    if sample_host is not None and a.mode == "fused":
        wh = None if inp.weight is None else inp.weight.cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(sample_host[0], sample_host[1], wh, w, red,
                                           a.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
