"""Benchmark of the fused softmax cross-entropy forward + gradient on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode MODE]
    python bench.py --configs-only          # one JSON line per configuration

A step is one pass of the whole hot path over one batch of synthetic logits
already resident in HBM: ce_forward (loss + gradient written over the
logits) followed by ce_backward with grad_output = 1 (the training call
pattern). Every step gets its own pristine copy of the batch (prepared
before the timed region), so no step reads a gradient left by another.
--mode nograd times the forward without the gradient (an evaluation pass);
--mode recompute keeps the logits and times the gradient recomputed from
them (ce_backward_recompute) after that forward.

The default workload is 1023 rows x V = 128256 fp32 logits, reduction
"sum" (the tt-mlir PR #9324 page's before/after shape). The one JSON line
printed holds rows/s over the K timed steps, the roofline of the forward
call (algorithmic bytes over its HIP-event-timed duration on the launch
stream) against 8 TB/s and against the in-place HBM ceiling that the
stream kernels (include/ce_stream.h) measure over the same bytes in the
same run, and the float64 oracle timed on the host cores. Unless
--no-configs, it also holds every configuration's cold timings (batch
restored and 1 GiB flushed through the caches before each launch):
median / min / p90 of the forward, the backward at grad_output 1 and 0.5,
and each one's fraction of 8 TB/s and of its measured ceiling.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "ce_1023x128256_f32"
DEFAULT_REDUCTION = {"ce_1023x128256_f32": "sum"}
PROFILES = os.path.join(ROOT, "profiles")


# The sources the fused cross-entropy kernels (and the launches ce_forward
# makes) are built from; the linear, vocabulary-shard and stream kernels
# live in other files and do not change them.
FUSED_SOURCES = ("ce_device.hpp", "ce_kernels.hpp", "ce_wide.hpp", "ce_launch.hpp",
                 "ce_launch_impl.hpp", "ce_plan.hpp", "ce_api.hip", "ce_inst_f32.hip",
                 "ce_inst_bf16.hip", "ce_inst_f32_wide.hip", "ce_inst_bf16_wide.hip")


def source_hash() -> str:
    """Hash of the fused kernels' HIP sources: counter-based traffic figures
    are valid only for the kernels they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "softmax_cross_entropy_amd", "csrc")
    for name in FUSED_SOURCES:
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


def linear_forward_bench(steps: int, warmup: int, rows: int = 4096, H: int = 4096,
                         V: int = 128256) -> None:
    """The linear layer fused with the cross-entropy without gradients (an
    evaluation step: loss, z-loss, token accuracy, argmax) at the language-model
    head shape: the matrix-core kernel that keeps the logits on chip
    (CE_F_LINEAR_ON_CHIP), the library GEMM path with fp32 logits (the
    default), and PyTorch eager
    (bf16 matmul, fp32 cross-entropy) under no_grad. Matrix-core roofline:
    2 rows V H flops per step against the bf16 dense peak."""
    import torch
    import torch.nn.functional as F
    import synth
    from softmax_cross_entropy_amd import _lib, linear_forward_raw

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    x = (torch.randn(rows, H, device=dev, generator=g) * 0.5).to(torch.bfloat16)
    w = (torch.randn(V, H, device=dev, generator=g) * (2.0 / H ** 0.5)).to(torch.bfloat16)
    t = synth.make_targets(rows, V, 7, rows // 20).to(dev)
    kw = dict(reduction="mean", grad=False, token_accuracy=True, argmax=True)

    def matrix_core():
        linear_forward_raw(x, w, t, flags=_lib.CE_F_LINEAR_ON_CHIP, **kw)

    def library():
        linear_forward_raw(x, w, t, **kw)

    def eager():
        with torch.no_grad():
            lg = (x @ w.t()).float()
            F.cross_entropy(lg, t, ignore_index=-100)
            lg.argmax(dim=1)

    res = {}
    for name, fn in (("matrix_core_kernel", matrix_core), ("library_gemm", library),
                     ("torch_eager", eager)):
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
    flops = 2.0 * rows * V * H
    tf = flops / (res["matrix_core_kernel"] * 1e-3) / 1e12
    print(json.dumps({
        "linear_forward": "linear layer fused with the cross-entropy, no gradients (loss, "
                          "token accuracy, argmax), mean, bf16 inputs",
        "config": {"rows": rows, "H": H, "V": V},
        "ms_per_step": res,
        "speedup_vs_library_gemm": res["library_gemm"] / res["matrix_core_kernel"],
        "speedup_vs_torch_eager": res["torch_eager"] / res["matrix_core_kernel"],
        "roofline": {"bound": "mfma", "achieved": tf, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tf / 2500.0, "flops_per_step": flops}}), flush=True)


def shard_bench(reps: int = 20, G: int = 8) -> None:
    """One device's share of the headline batch split over G vocabulary shards
    (1023 rows x 128256 / G columns of fp32, reduction sum): stage 1 on its
    columns, then stage 2 with the G shards' partials (gathered beforehand,
    as the all-gather of a multi-device run would), timed cold per call
    pair; next to the fused kernel on the same columns. JSON line."""
    import torch
    import synth
    from softmax_cross_entropy_amd import _lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    flush = Flusher(dev)
    w = synth.WORKLOADS["ce_1023x128256_f32"]
    inp = synth.make_inputs(w, dev)
    rows, V = w.rows, w.V
    Vl = V // G
    slices = [inp.logits[:, g * Vl:(g + 1) * Vl].contiguous() for g in range(G)]
    t = inp.target
    parts = torch.zeros((G, rows, 32), dtype=torch.uint8, device=dev)
    for g in range(G):
        _lib.check(_lib.ce_shard_partials(slices[g].data_ptr(), _lib.CE_F32, rows, Vl, Vl, g * Vl,
                                          V, t.data_ptr(), 0, -100, 0.0, 0.0,
                                          parts[g].data_ptr(), s), "ce_shard_partials")
    loss = torch.empty((), device=dev)
    wsb = _lib.ce_shard_workspace_bytes(rows)
    ws = torch.zeros((wsb,), dtype=torch.uint8, device=dev)
    fws_b = _lib.ce_workspace_bytes(rows, Vl, _lib.CE_F32, _lib.CE_F_GRAD)
    fws = torch.zeros((fws_b,), dtype=torch.uint8, device=dev)
    buf = torch.empty_like(slices[0])

    def sharded():
        _lib.check(_lib.ce_shard_partials(buf.data_ptr(), _lib.CE_F32, rows, Vl, Vl, 0, V,
                                          t.data_ptr(), 0, -100, 0.0, 0.0, parts[0].data_ptr(),
                                          s), "ce_shard_partials")
        _lib.check(_lib.ce_shard_finish(buf.data_ptr(), _lib.CE_F32, rows, Vl, Vl, 0, V,
                                        t.data_ptr(), 0, -100, 0.0, 0.0, 0.0, _lib.CE_RED_SUM, 0,
                                        parts.data_ptr(), G, loss.data_ptr(), 0, 0, 0, 0,
                                        ws.data_ptr(), wsb, s), "ce_shard_finish")

    def fused():  # the single-device kernel on the same columns (its own row of V_l classes)
        _lib.check(_lib.ce_forward(buf.data_ptr(), _lib.CE_F32, rows, Vl, Vl, t.data_ptr(), 0,
                                   -100, 0.0, 0.0, 0.0, _lib.CE_RED_SUM, _lib.CE_F_GRAD,
                                   loss.data_ptr(), 0, 0, 0, 0, 0, fws.data_ptr(), fws_b, s),
                   "ce_forward")

    def stage1():
        _lib.check(_lib.ce_shard_partials(buf.data_ptr(), _lib.CE_F32, rows, Vl, Vl, 0, V,
                                          t.data_ptr(), 0, -100, 0.0, 0.0, parts[0].data_ptr(),
                                          s), "ce_shard_partials")

    res = {}
    for name, fn in (("shard", sharded), ("stage1_alone", stage1), ("fused_same_columns", fused)):
        ts = []
        for i in range(reps + 2):
            buf.copy_(slices[0])
            flush(stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        res[name] = _stats(ts)
    n_counted = int((t != -100).sum().item())
    one_pass = rows * Vl * 4
    print(json.dumps({
        "shard": f"one of {G} vocabulary shards of the 1023 x 128256 fp32 batch (sum)",
        "rows": rows, "V_local": Vl, "V_total": V,
        "us": {k: {kk: round(vv, 2) for kk, vv in v.items()} for k, v in res.items()},
        "ratio_to_fused": res["shard"]["median"] / res["fused_same_columns"]["median"],
        "GBps_three_passes": (2 * one_pass + n_counted * Vl * 4) / (res["shard"]["median"] * 1e-6)
                             / 1e9}), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_host, t_host, weight_host, w, reduction, budget_s=12.0):
    """Time the float64 oracle, as it is, on a bounded sample of the batch's
    rows: once in this process alone, once over threads that each run it on
    64-row chunks (numpy's array loops release the GIL), one thread per host
    core this process may use (at most 16). The threaded rate is the
    baseline; `cores` is the number of threads it used."""
    import concurrent.futures as cf
    import numpy as np
    from oracle import rows_forward, summarize_targets

    summ = summarize_targets(t_host, w.V, -100, weight_host, reduction)
    rows_per_call = 64
    n = x_host.shape[0]

    def call(a):
        b = min(n, a + rows_per_call)
        rows_forward(x_host[a:b], t_host[a:b], V=w.V, alpha=summ.alpha, beta=summ.beta,
                     weight=weight_host, label_smoothing=w.label_smoothing,
                     lse_square_scale=w.lse_square_scale, softcap=w.softcap or None,
                     want_grad=True)
        return b - a

    def run(workers, budget):
        done = 0
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(workers) as ex:
            while time.perf_counter() - t0 < budget:
                done += sum(ex.map(call, range(0, n, rows_per_call)))
        return done / (time.perf_counter() - t0), done

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    single, n1 = run(1, budget_s / 2)
    threaded, nt = run(cores, budget_s / 2)
    digest = hashlib.sha256(np.ascontiguousarray(x_host).tobytes() +
                            np.ascontiguousarray(t_host).tobytes()).hexdigest()[:16]
    return {"value": threaded, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {n} rows of the {w.name} batch (inputs sha256 {digest}), "
                      f"loss and gradient in float64, over {cores} threads of 64-row calls "
                      f"for {budget_s / 2:.0f} s ({nt} rows); one thread alone: "
                      f"{single:.1f} rows/s ({n1} rows)",
            "single_thread_value": single,
            "host_cpu": _cpu_model(), "host_cores_available": len(os.sched_getaffinity(0))}


# ---------------------------------------------------------------------------
# Per-config measurement on cold buffers: before each timed launch the batch
# is restored from a pristine device copy and 1 GiB is read through the
# caches (the flush stream kernel), so the launch reads its logits from HBM.
# ---------------------------------------------------------------------------

CONFIGS = (  # (label, workload, reduction)
    ("C1", "ce_64x4096_f32", "mean"),
    ("C2", "ce_4096x32768_bf16", "mean"),
    ("C3", "ce_1023x128256_f32", "sum"),
    ("C3none", "ce_1023x128256_f32", "none"),
    ("C4", "ce_4096x131072_bf16_opts", "mean"),
    ("C5", "ce_16384x262144_bf16", "mean"),
    ("C5b", "ce_512x262144_bf16_allignored", "mean"),
)


class Case:
    """One workload's inputs resident on the GPU and the raw forward/backward calls."""

    def __init__(self, w, red, flags_extra=0, mode="fused", dev=None):
        import torch
        from softmax_cross_entropy_amd import _lib
        from softmax_cross_entropy_amd.functional import _workspace
        self.w, self.red, self.mode = w, red, mode
        self.dev = dev
        self.stream = torch.cuda.current_stream(dev)
        self.inp = synth_inputs(w, dev)
        t_host = self.inp.target.cpu().numpy()
        self.n_counted = int(((t_host != -100) & (t_host >= 0) & (t_host < w.V)).sum())
        self.dt = _lib.dtype_code(w.dtype)
        self.flags = (_lib.CE_F_GRAD if mode == "fused" else 0) | flags_extra
        rows, V = w.rows, w.V
        f32 = dict(device=dev, dtype=torch.float32)
        self.loss = torch.empty((rows,) if red == "none" else (), **f32)
        self.z_loss = torch.empty_like(self.loss) if w.want_z_loss else None
        self.acc = torch.empty_like(self.loss) if w.want_accuracy else None
        self.arg = torch.empty((rows,), device=dev, dtype=torch.int64) if w.want_argmax else None
        self.stats = torch.empty((rows, 2), **f32) if mode == "recompute" else None
        self.ws_bytes = _lib.ce_workspace_bytes(rows, V, self.dt, self.flags)
        self.ws = _workspace(dev, self.ws_bytes)
        self.red_code = _lib.REDUCTION_CODES[red]
        P = self.P
        x = self.inp.logits
        self.path = _lib.PATH_NAMES[_lib.ce_plan_path(P(x), self.dt, rows, V, x.stride(0),
                                                      P(self.inp.weight), w.label_smoothing,
                                                      self.flags)]

    @staticmethod
    def P(t):
        return 0 if t is None else t.data_ptr()

    def fwd(self, buf):
        from softmax_cross_entropy_amd import _lib
        w, P = self.w, self.P
        st = _lib.ce_forward(P(buf), self.dt, w.rows, w.V, buf.stride(0), P(self.inp.target),
                             P(self.inp.weight), -100, w.label_smoothing, w.lse_square_scale,
                             w.softcap, self.red_code, self.flags, P(self.loss), P(self.z_loss),
                             P(self.acc), P(self.arg), 0, P(self.stats), P(self.ws),
                             self.ws_bytes, self.stream.cuda_stream)
        if st:
            raise _lib.CEError(st, "ce_forward")

    def bwd(self, buf, go, out=None):
        from softmax_cross_entropy_amd import _lib
        w, P = self.w, self.P
        if self.mode == "recompute":
            st = _lib.ce_backward_recompute(P(buf), self.dt, w.rows, w.V, buf.stride(0),
                                            P(self.inp.target), P(self.inp.weight), -100,
                                            w.label_smoothing, w.lse_square_scale, w.softcap,
                                            self.red_code, P(self.stats), P(go), 0, P(out),
                                            out.stride(0), P(self.ws), self.ws_bytes,
                                            self.stream.cuda_stream)
        else:
            st = _lib.ce_backward(P(buf), self.dt, w.rows, w.V, buf.stride(0), P(go), 0,
                                  self.stream.cuda_stream)
        if st:
            raise _lib.CEError(st, "backward")


def synth_inputs(w, dev):
    import synth
    return synth.make_inputs(w, dev)


class Flusher:
    """Reads 1 GiB through the caches (the stream kernels' flush), so the next
    launch finds none of its data in L2 or the Infinity Cache."""

    def __init__(self, dev):
        import torch
        self.buf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def __call__(self, stream):
        from softmax_cross_entropy_amd import _lib
        _lib.check(_lib.ce_stream_run(_lib.CE_STREAM_FLUSH, 4, 0, self.buf.data_ptr(),
                                      self.buf.numel() * 4, 0, self.sink.data_ptr(),
                                      stream.cuda_stream), "flush")


def _stats(us):
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return {"median": float(np.median(a)), "min": float(a.min()),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def ceilings(nbytes, dev, flush, reps=5):
    """HBM ceilings over `nbytes` measured with the stream kernels (each launch
    cold, after the flush): in-place read-then-write, copy, read, write; the
    best over a few chunk shapes and grids. GB/s of the best launch, and of
    the median launch of that shape."""
    import torch
    from softmax_cross_entropy_amd import _lib
    stream = torch.cuda.current_stream(dev)
    nbytes = nbytes // 16 * 16
    a = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.zeros_like(a)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    out = {}
    for kind, name, moved in ((_lib.CE_STREAM_INPLACE, "inplace", 2), (_lib.CE_STREAM_COPY, "copy", 2),
                              (_lib.CE_STREAM_READ, "read", 1), (_lib.CE_STREAM_WRITE, "write", 1)):
        best = None
        for cfg in (2, 5, 7):  # 256 x 16, 512 x 16, 1024 x 8 vectors per chunk
            res = _lib.ce_stream_resident(kind, cfg)
            for grid in (0, res):
                ts = []
                for _ in range(reps):
                    flush(stream)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    dst = a.data_ptr() if kind in (_lib.CE_STREAM_INPLACE, _lib.CE_STREAM_WRITE) else (
                        b.data_ptr() if kind == _lib.CE_STREAM_COPY else 0)
                    src = a.data_ptr() if kind in (_lib.CE_STREAM_COPY, _lib.CE_STREAM_READ) else 0
                    _lib.check(_lib.ce_stream_run(kind, cfg, dst, src, nbytes, grid,
                                                  sink.data_ptr(), stream.cuda_stream), name)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3)
                st = _stats(ts)
                if best is None or st["min"] < best["min"]:
                    blk, nreg = _lib.ce_stream_config(cfg)
                    best = dict(st, shape=f"{blk}x{nreg}", grid="one per chunk" if grid == 0 else grid)
        best["GBps"] = moved * nbytes / (best["min"] * 1e-6) / 1e9
        best["GBps_median"] = moved * nbytes / (best["median"] * 1e-6) / 1e9
        out[name] = best
    del a, b
    return out


def measure_config(label, wname, red, dev, flush, reps, ceil_reps=5):
    """Cold per-launch timings of one workload: the forward (+ gradient) call,
    the backward at grad_output 1 (exits at once) and 0.5 (a pass over the
    gradient), with the roofline of the forward against 8 TB/s and against the
    in-place ceiling measured over the same bytes in the same run."""
    import torch
    import synth
    w = synth.WORKLOADS[wname]
    c = Case(w, red, dev=dev)
    stream = c.stream
    pristine = c.inp.logits
    buf = torch.empty_like(pristine)
    go1 = torch.ones((), device=dev, dtype=torch.float32)
    go05 = torch.full((), 0.5, device=dev, dtype=torch.float32)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    fwd_us, b1_us, b05_us = [], [], []
    for i in range(reps + 1):  # the first round warms up
        for go, sink in ((go1, b1_us), (go05, b05_us)):
            buf.copy_(pristine)
            flush(stream)
            e = [ev() for _ in range(4)]
            e[0].record(stream)
            c.fwd(buf)
            e[1].record(stream)
            flush(stream)
            e[2].record(stream)
            c.bwd(buf, go)
            e[3].record(stream)
            torch.cuda.synchronize()
            if i > 0:
                if go is go1:
                    fwd_us.append(e[0].elapsed_time(e[1]) * 1e3)
                sink.append(e[2].elapsed_time(e[3]) * 1e3)
    alg = algorithmic_bytes(w, red, c.n_counted)
    f = _stats(fwd_us)
    nbytes = w.rows * w.V * w.elem_bytes
    ceil = ceilings(nbytes, dev, flush, ceil_reps)
    bound = "write" if c.n_counted == 0 else "inplace"
    ce = ceil[bound]
    achieved = alg / (f["median"] * 1e-6) / 1e9
    rec = {
        "workload": w.name, "reduction": red, "path": c.path, "rows": w.rows, "V": w.V,
        "dtype": "f32" if w.elem_bytes == 4 else "bf16",
        "forward_us": f, "backward_go1_us": _stats(b1_us), "backward_go05_us": _stats(b05_us),
        "rows_per_s": w.rows / (f["median"] * 1e-6),
        "algorithmic_bytes": alg,
        "roofline": {"bound": "hbm", "achieved_GBps": achieved, "peak_GBps": HBM_PEAK_GBPS,
                     "frac": achieved / HBM_PEAK_GBPS,
                     "ceiling": bound, "ceiling_GBps": ce["GBps_median"],
                     "frac_of_ceiling": achieved / ce["GBps_median"],
                     "best_launch_frac": alg / (f["min"] * 1e-6) / 1e9 / HBM_PEAK_GBPS},
        "ceilings": {k: {"GBps": v["GBps"], "GBps_median": v["GBps_median"], "shape": v["shape"],
                         "grid": v["grid"]} for k, v in ceil.items()},
    }
    del c, buf, pristine
    torch.cuda.empty_cache()
    return label, rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--reduction", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the cold per-config measurements (faster; for profiling runs)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the stream-kernel ceilings of the headline line (profiling runs)")
    ap.add_argument("--config-reps", type=int, default=10,
                    help="cold launches per config and per backward variant")
    ap.add_argument("--configs-only", action="store_true",
                    help="print one JSON line per config (C1..C5b) and exit")
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
    ap.add_argument("--forward-only", action="store_true",
                    help="--linear: the forward without gradients (matrix-core kernel against "
                         "the library GEMM path and PyTorch eager)")
    ap.add_argument("--chunk-rows", type=int, default=0,
                    help="--linear: rows per chunk (0: the library's default)")
    ap.add_argument("--sweep", action="store_true",
                    help="context sweep over V at the Liger benchmark shape, this library "
                         "against PyTorch eager F.cross_entropy (JSON line per V), then exit")
    ap.add_argument("--shard", action="store_true",
                    help="one of 8 vocabulary shards of the default batch: the two shard calls "
                         "against the fused kernel on the same columns (JSON line), then exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the fused kernel's HBM traffic from two rocprofv3 --pmc "
                         "counter_collection.csv files of this benchmark, then exit")
    a = ap.parse_args(argv)
    if a.traffic:
        write_traffic(a.workload, *a.traffic)
        return 0

    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported: the library runs "
              "on one GPU (the path would shard by rows, with no communication between GPUs "
              "on the hot path).", file=sys.stderr)
        return 2

    if a.linear:
        if a.forward_only:
            linear_forward_bench(a.steps, a.warmup)
        else:
            linear_bench(a.steps, a.warmup, chunk_rows=a.chunk_rows)
        return 0

    if a.sweep:
        from softmax_cross_entropy_amd import _lib
        sweep(a.steps, a.warmup, _lib.CE_F_SHAPE_ALT if a.alt_shape else 0)
        return 0

    if a.shard:
        shard_bench()
        return 0

    import torch
    import synth
    from softmax_cross_entropy_amd import _lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = Flusher(dev)

    if a.configs_only:
        for label, wname, red in CONFIGS:
            lab, rec = measure_config(label, wname, red, dev, flush, a.config_reps)
            print(json.dumps(dict(config=lab, **rec)), flush=True)
        return 0

    w = synth.WORKLOADS[a.workload]
    red = a.reduction or DEFAULT_REDUCTION.get(w.name, w.reductions[0])
    flags = {"auto": 0, "fused": _lib.CE_F_FORCE_FUSED, "splitv": _lib.CE_F_FORCE_SPLITV,
             "scalar": _lib.CE_F_FORCE_SCALAR}[a.path]
    if a.alt_shape:
        flags |= _lib.CE_F_SHAPE_ALT
    c = Case(w, red, flags, a.mode, dev)
    stream = c.stream
    rows, V = w.rows, w.V
    sample_host = None
    if not a.no_cpu_baseline and a.mode == "fused":
        x = c.inp.logits[:256].detach().cpu()
        sample_host = (x.view(torch.int16).numpy().view("uint16") if x.dtype == torch.bfloat16
                       else x.numpy(), c.inp.target[:256].cpu().numpy())
    # every step on its own pristine copy of the batch, made before the timed region
    nbuf = a.warmup + a.steps
    bufs = [c.inp.logits.clone() for _ in range(nbuf)]
    go = torch.ones((), device=dev, dtype=torch.float32)
    gbuf = torch.empty_like(c.inp.logits) if a.mode == "recompute" else None

    def step(b):
        c.fwd(b)
        if a.mode != "nograd":
            c.bwd(b, go, gbuf)

    # The timed kernel: the forward call, or the recomputing backward.
    timed_first = a.mode != "recompute"
    for i in range(a.warmup):
        step(bufs[i])
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
            c.fwd(b)
            ev[i][1].record(stream)
            if a.mode != "nograd":
                c.bwd(b, go, gbuf)
        else:
            c.fwd(b)
            ev[i][0].record(stream)
            c.bwd(b, go, gbuf)
            ev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    kern_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    kernel_ms = sum(kern_us) / len(kern_us) / 1e3
    ms_per_step = total_ms / a.steps
    del bufs

    alg = algorithmic_bytes(w, red, c.n_counted, a.mode)
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    kernel_key = "ce_fused" if c.path == "fused" else f"ce_{c.path}"
    traffic = traffic_from_profiles(w.name, kernel_key) if a.mode == "fused" else None
    nbytes = rows * V * w.elem_bytes
    ceil = None if a.no_ceilings else ceilings(nbytes, dev, flush)
    # the stream kernel that moves the same bytes: in place, or read only
    # for the forward without the gradient
    ceil_kind = "read" if a.mode == "nograd" else "inplace"
    ce = ceil[ceil_kind] if ceil else None
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
                   "reduction": red, "path": c.path,
                   "layout": "alternative" if a.alt_shape else "default",
                   "label_smoothing": w.label_smoothing, "softcap": w.softcap,
                   "lse_square_scale": w.lse_square_scale, "class_weights": w.weights,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel_ms": kernel_ms, "kernel_us_stats": _stats(kern_us),
                     "algorithmic_bytes": alg,
                     f"ceiling_{ceil_kind}_GBps": ce["GBps_median"] if ce else None,
                     "frac_of_ceiling": achieved / ce["GBps_median"] if ce else None},
        "ceilings_GBps": {k: {"best": v["GBps"], "median": v["GBps_median"], "shape": v["shape"]}
                          for k, v in ceil.items()} if ceil else None,
    }
    if not a.no_configs and a.mode == "fused":
        out["configs"] = {}
        for label, wname, cred in CONFIGS:
            lab, rec = measure_config(label, wname, cred, dev, flush, a.config_reps, ceil_reps=3)
            out["configs"][lab] = {
                "workload": rec["workload"], "reduction": rec["reduction"], "path": rec["path"],
                "forward_us": {k: round(v, 2) for k, v in rec["forward_us"].items()},
                "backward_go1_us_median": round(rec["backward_go1_us"]["median"], 2),
                "backward_go05_us_median": round(rec["backward_go05_us"]["median"], 2),
                "rows_per_s": rec["rows_per_s"],
                "GBps": round(rec["roofline"]["achieved_GBps"], 1),
                "frac_of_8TBps": round(rec["roofline"]["frac"], 4),
                "ceiling": rec["roofline"]["ceiling"],
                "ceiling_GBps": round(rec["roofline"]["ceiling_GBps"], 1),
                "frac_of_ceiling": round(rec["roofline"]["frac_of_ceiling"], 4)}
    if sample_host is not None:
        wh = None if c.inp.weight is None else c.inp.weight.cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(sample_host[0], sample_host[1], wh, w, red,
                                           a.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
