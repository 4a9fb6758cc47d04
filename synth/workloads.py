"""The synthetic workloads and their seeded generators.

Shapes follow the pages' workloads: the Liger-Kernel cross-entropy profile's
benchmark sweep (B=8, T=512 rows, bf16, V from 4096 to 131072) and the
tt-mlir PR #9324 before/after table (rows=1023, C=128256, f32). Values are
Gaussian logits, uniform targets with a fixed share set to ignore_index.

Recipe (deterministic for a given device type):
  * logits: torch.Generator(device).manual_seed(seed); rows are drawn in
    blocks of ``GEN_BLOCK`` rows, each block with torch.randn(float32) * sigma
    from a generator re-seeded with seed * 1_000_003 + block; bf16 logits
    are the float32 draws rounded to nearest-even by torch.
  * targets: CPU generator seeded with seed + 1: torch.randint(0, V); then
    round(frac * rows) rows, picked by torch.randperm, set to ignore_index.
  * class weights: CPU generator seeded with seed + 2: 0.5 + 1.5 * rand(V).
  * large-logit rows: 10 counted rows picked by a CPU generator seeded with
    seed + 3; the first five get +80 at their target, the others +80 at a
    drawn column different from the target.
  * all-ignored rows with non-finite logits: row r holds NaN (r % 4 == 0),
    +inf (1), -inf (2), or N(0,1) draws with one NaN, one +inf and one -inf
    at drawn columns (3); every target is ignore_index.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

GEN_BLOCK = 1024
IGNORE = -100


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    V: int
    dtype: torch.dtype
    sigma: float
    seed: int
    ignore_frac: float = 0.0
    weights: bool = False
    label_smoothing: float = 0.0
    softcap: float = 0.0
    lse_square_scale: float = 0.0
    reductions: tuple = ("mean",)
    spikes: int = 0
    all_ignored_nonfinite: bool = False
    want_accuracy: bool = False
    want_argmax: bool = False
    want_z_loss: bool = False

    @property
    def n_ignored(self) -> int:
        if self.all_ignored_nonfinite:
            return self.rows
        return int(round(self.ignore_frac * self.rows))

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == torch.bfloat16 else 4


WORKLOADS = {
    "ce_64x4096_f32": Workload("ce_64x4096_f32", 64, 4096, torch.float32, 1.0, 101,
                               ignore_frac=0.10, reductions=("mean",)),
    "ce_4096x32768_bf16": Workload("ce_4096x32768_bf16", 4096, 32768, torch.bfloat16, 2.0, 102,
                                   ignore_frac=0.05, reductions=("mean",), want_accuracy=True,
                                   want_argmax=True),
    "ce_1023x128256_f32": Workload("ce_1023x128256_f32", 1023, 128256, torch.float32, 1.0, 103,
                                   ignore_frac=0.02, reductions=("sum", "none"), spikes=10),
    "ce_4096x131072_bf16_opts": Workload("ce_4096x131072_bf16_opts", 4096, 131072, torch.bfloat16,
                                         3.0, 104, weights=True, label_smoothing=0.1,
                                         softcap=30.0, lse_square_scale=1e-4,
                                         reductions=("mean",), want_z_loss=True),
    "ce_16384x262144_bf16": Workload("ce_16384x262144_bf16", 16384, 262144, torch.bfloat16, 1.0,
                                     105, ignore_frac=0.01, reductions=("mean",)),
    "ce_512x262144_bf16_allignored": Workload("ce_512x262144_bf16_allignored", 512, 262144,
                                              torch.bfloat16, 1.0, 1055, reductions=("mean",),
                                              all_ignored_nonfinite=True),
    # one GPU's slice of the 1023 x 128256 batch split over 8 vocabulary shards
    "ce_1023x16032_f32_shard": Workload("ce_1023x16032_f32_shard", 1023, 16032, torch.float32,
                                        1.0, 107, ignore_frac=0.02, reductions=("sum",)),
}


def _cpu_gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def make_logits(rows: int, V: int, dtype: torch.dtype, sigma: float, seed: int,
                device="cpu", row_stride: Optional[int] = None) -> torch.Tensor:
    """Gaussian logits N(0, sigma^2), (rows, V) view of a (rows, row_stride) buffer."""
    stride = V if row_stride is None else row_stride
    dev = torch.device(device)
    buf = torch.empty((rows, stride), dtype=dtype, device=dev)
    for b0 in range(0, rows, GEN_BLOCK):
        b1 = min(rows, b0 + GEN_BLOCK)
        g = torch.Generator(device=dev)
        g.manual_seed(seed * 1_000_003 + b0 // GEN_BLOCK)
        blk = torch.randn((b1 - b0, stride), dtype=torch.float32, device=dev, generator=g)
        blk.mul_(sigma)
        buf[b0:b1].copy_(blk)
        del blk
    return buf[:, :V]


def make_targets(rows: int, V: int, seed: int, n_ignored: int) -> torch.Tensor:
    g = _cpu_gen(seed + 1)
    t = torch.randint(0, V, (rows,), generator=g, dtype=torch.int64)
    if n_ignored:
        idx = torch.randperm(rows, generator=g)[:n_ignored]
        t[idx] = IGNORE
    return t


@dataclass
class Inputs:
    logits: torch.Tensor
    target: torch.Tensor
    weight: Optional[torch.Tensor]
    spike_rows: list = field(default_factory=list)


def _place_spikes(x: torch.Tensor, t: torch.Tensor, seed: int, count: int) -> list:
    g = _cpu_gen(seed + 3)
    rows, V = x.shape
    counted = torch.nonzero(t != IGNORE).flatten()
    pick = counted[torch.randperm(counted.numel(), generator=g)[:count]].tolist()
    for j, r in enumerate(pick):
        y = int(t[r])
        if j < count // 2:
            col = y
        else:
            col = int(torch.randint(0, V - 1, (1,), generator=g))
            col = col + 1 if col >= y else col
        x[r, col] = 80.0
    return pick


def _fill_nonfinite(x: torch.Tensor, seed: int) -> None:
    g = _cpu_gen(seed + 4)
    rows, V = x.shape
    x[0::4] = float("nan")
    x[1::4] = float("inf")
    x[2::4] = float("-inf")
    for r in range(3, rows, 4):
        cols = torch.randperm(V, generator=g)[:3].tolist()
        x[r, cols[0]] = float("nan")
        x[r, cols[1]] = float("inf")
        x[r, cols[2]] = float("-inf")


def make_inputs(w: Workload, device="cpu", row_stride: Optional[int] = None) -> Inputs:
    """All inputs of a workload, on ``device`` (targets and weights included)."""
    x = make_logits(w.rows, w.V, w.dtype, w.sigma, w.seed, device, row_stride)
    t = make_targets(w.rows, w.V, w.seed, 0 if w.all_ignored_nonfinite else w.n_ignored)
    if w.all_ignored_nonfinite:
        t.fill_(IGNORE)
        _fill_nonfinite(x, w.seed)
    spikes = _place_spikes(x, t, w.seed, w.spikes) if w.spikes else []
    weight = None
    if w.weights:
        weight = 0.5 + 1.5 * torch.rand(w.V, generator=_cpu_gen(w.seed + 2), dtype=torch.float32)
        weight = weight.to(device)
    return Inputs(x, t.to(device), weight, spikes)
