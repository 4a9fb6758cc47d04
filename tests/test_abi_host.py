"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, shares the process's HIP runtime, and rejects invalid
arguments before enqueuing anything (no GPU needed: validation runs first).
"""

import os
import re
import subprocess
import sys

import pytest

from softmax_cross_entropy_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            src = open(os.path.join(INCLUDE, h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names.update(re.findall(r"\b(ce_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert names == sorted(_lib.SYMBOLS)
    h = _lib.lib()
    for n in names:
        assert hasattr(h, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(set(re.findall(r" T (ce_\w+)", out)))
    assert exported == names


def test_single_hip_runtime_in_process():
    _lib.lib()
    maps = open("/proc/self/maps").read()
    libs = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(libs) == 1, libs


def test_missing_library_fails_loudly(tmp_path):
    code = (
        "import softmax_cross_entropy_amd._lib as L\n"
        f"L.LIB_PATH = {str(tmp_path / 'nope.so')!r}\n"
        "try:\n"
        "    L.lib()\n"
        "except RuntimeError as e:\n"
        "    print('RAISED', e)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "RAISED" in r.stdout and "not built" in r.stdout


def test_status_strings():
    for s in range(-9, 1):
        assert _lib.ce_status_string(s) and _lib.ce_status_string(s) != "unknown status"
    assert _lib.ce_status_string(42) == "unknown status"


FAKE = 1 << 20  # never dereferenced: every call below fails validation first


def _fwd(**kw):
    a = dict(logits=FAKE, dtype=_lib.CE_F32, rows=4, V=16, row_stride=16, target=FAKE, weight=0,
             ignore_index=-100, label_smoothing=0.0, lse_square_scale=0.0, softcap=0.0,
             reduction=_lib.CE_RED_MEAN, flags=0, loss=FAKE, z_loss=0, token_accuracy=0,
             argmax=0, counts=0, row_stats=0, workspace=0, workspace_bytes=0, stream=0)
    a.update(kw)
    return _lib.ce_forward(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), _lib.CE_E_DTYPE),
    (dict(rows=-1), _lib.CE_E_SHAPE),
    (dict(V=0), _lib.CE_E_SHAPE),
    (dict(row_stride=15), _lib.CE_E_SHAPE),
    (dict(V=1 << 31, row_stride=1 << 31), _lib.CE_E_SHAPE),
    (dict(reduction=3), _lib.CE_E_PARAM),
    (dict(label_smoothing=1.5), _lib.CE_E_PARAM),
    (dict(label_smoothing=float("nan")), _lib.CE_E_PARAM),
    (dict(softcap=-1.0), _lib.CE_E_PARAM),
    (dict(softcap=float("inf")), _lib.CE_E_PARAM),
    (dict(lse_square_scale=float("nan")), _lib.CE_E_PARAM),
    (dict(lse_square_scale=-1.0), _lib.CE_E_PARAM),
    (dict(loss=0), _lib.CE_E_NULL),
    (dict(logits=0), _lib.CE_E_NULL),
    (dict(target=0), _lib.CE_E_NULL),
    (dict(workspace=0, workspace_bytes=1 << 20), _lib.CE_E_WORKSPACE),
    (dict(workspace=FAKE + 8, workspace_bytes=1 << 20), _lib.CE_E_WORKSPACE),
    (dict(workspace=FAKE, workspace_bytes=64), _lib.CE_E_WORKSPACE),
])
def test_forward_validation(kw, status):
    assert _fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), _lib.CE_E_DTYPE),
    (dict(rows=-3), _lib.CE_E_SHAPE),
    (dict(row_stride=3), _lib.CE_E_SHAPE),
    (dict(grad_output=0), _lib.CE_E_NULL),
    (dict(grad=0), _lib.CE_E_NULL),
    (dict(rows=0, grad=0), _lib.CE_OK),
])
def test_backward_validation(kw, status):
    a = dict(grad=FAKE, dtype=_lib.CE_BF16, rows=4, V=16, row_stride=16, grad_output=FAKE,
             per_row=0, stream=0)
    a.update(kw)
    assert _lib.ce_backward(**a) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), _lib.CE_E_DTYPE),
    (dict(rows=-1), _lib.CE_E_SHAPE),
    (dict(row_stride=15), _lib.CE_E_SHAPE),
    (dict(grad_stride=15), _lib.CE_E_SHAPE),
    (dict(grad=FAKE, grad_stride=32), _lib.CE_E_SHAPE),   # in place needs the logits' stride
    (dict(reduction=5), _lib.CE_E_PARAM),
    (dict(label_smoothing=-0.5), _lib.CE_E_PARAM),
    (dict(softcap=float("nan")), _lib.CE_E_PARAM),
    (dict(grad_output=0), _lib.CE_E_NULL),
    (dict(row_stats=0), _lib.CE_E_NULL),
    (dict(grad=0), _lib.CE_E_NULL),
    (dict(logits=0), _lib.CE_E_NULL),
    (dict(workspace=0), _lib.CE_E_WORKSPACE),
    (dict(workspace=FAKE + 16), _lib.CE_E_WORKSPACE),
    (dict(workspace_bytes=128), _lib.CE_E_WORKSPACE),
    (dict(rows=0, logits=0, grad=0, row_stats=0), _lib.CE_OK),
])
def test_backward_recompute_validation(kw, status):
    a = dict(logits=FAKE, dtype=_lib.CE_F32, rows=4, V=16, row_stride=16, target=FAKE, weight=0,
             ignore_index=-100, label_smoothing=0.0, lse_square_scale=0.0, softcap=0.0,
             reduction=_lib.CE_RED_MEAN, row_stats=FAKE, grad_output=FAKE, per_row=0,
             grad=FAKE + 4096, grad_stride=16, workspace=FAKE, workspace_bytes=256, stream=0)
    a.update(kw)
    assert _lib.ce_backward_recompute(**a) == status


def test_workspace_bytes():
    ws = _lib.ce_workspace_bytes
    assert ws(4, 16, 9, 0) == 0
    assert ws(-1, 16, 0, 0) == 0
    base = ws(0, 16, _lib.CE_F32, 0)
    assert base >= 256 and base % 256 == 0
    # header + three per-row arrays, each rounded to 256 bytes
    assert ws(1023, 16384, _lib.CE_F32, 0) == 256 + 3 * 4096
    # rows of 4 K to 16 K vectors on a pair of workgroups add two 64-byte
    # exchange slots per row
    assert ws(1023, 32768, _lib.CE_F32, 0) == 256 + 3 * 4096 + 1023 * 128 + 128
    # quarter rows (rows of 16 K to 32 K vectors) add four 64-byte exchange slots
    # per row, the row pair of the alternative layout two (rounded to 256 bytes)
    assert ws(1023, 128256, _lib.CE_F32, 0) == 256 + 3 * 4096 + 1023 * 256
    assert (ws(1023, 128256, _lib.CE_F32, _lib.CE_F_SHAPE_ALT)
            == 256 + 3 * 4096 + 1023 * 128 + 128)
    # forced split-V adds the (rows, chunks) partials (32 bytes each)
    s = ws(64, 4096, _lib.CE_F32, _lib.CE_F_FORCE_SPLITV)
    assert s == 256 + 3 * 256 + 64 * 4 * 32


@pytest.mark.parametrize("dtype,V,rows,path", [
    (_lib.CE_F32, 4096, 64, _lib.CE_PATH_FUSED),
    (_lib.CE_F32, 128256, 1023, _lib.CE_PATH_FUSED),
    (_lib.CE_BF16, 262144, 16384, _lib.CE_PATH_FUSED),
    (_lib.CE_BF16, 131072, 4096, _lib.CE_PATH_FUSED),
    (_lib.CE_F32, 1 << 20, 64, _lib.CE_PATH_SPLITV),   # row larger than one CU holds
    (_lib.CE_BF16, 262144, 8, _lib.CE_PATH_SPLITV),    # too few rows to fill the GPU
])
def test_plan_paths(dtype, V, rows, path):
    assert _lib.ce_plan_path(FAKE, dtype, rows, V, V, 0, 0.0, 0) == path


def test_plan_unaligned_and_forced():
    P = _lib.ce_plan_path
    assert P(FAKE + 4, _lib.CE_F32, 8, 64, 64, 0, 0.0, 0) == _lib.CE_PATH_SCALAR
    assert P(FAKE, _lib.CE_F32, 8, 63, 63, 0, 0.0, 0) == _lib.CE_PATH_SCALAR      # row stride
    assert P(FAKE, _lib.CE_F32, 8, 63, 64, 0, 0.0, 0) == _lib.CE_PATH_FUSED
    assert P(FAKE, _lib.CE_F32, 8, 64, 64, FAKE + 4, 0.1, 0) == _lib.CE_PATH_SCALAR  # weights
    assert P(FAKE, _lib.CE_F32, 8, 64, 64, FAKE + 4, 0.0, 0) == _lib.CE_PATH_FUSED
    assert P(FAKE, _lib.CE_F32, 8, 64, 64, 0, 0.0, _lib.CE_F_FORCE_SPLITV) == _lib.CE_PATH_SPLITV
    assert P(FAKE, _lib.CE_F32, 8, 64, 64, 0, 0.0, _lib.CE_F_FORCE_SCALAR) == _lib.CE_PATH_SCALAR
    assert P(FAKE, 5, 8, 64, 64, 0, 0.0, 0) == _lib.CE_E_DTYPE
    assert P(FAKE, _lib.CE_F32, 8, 64, 32, 0, 0.0, 0) == _lib.CE_E_SHAPE


def test_python_layer_rejects_rank1_and_cpu_tensors():
    import torch
    import softmax_cross_entropy_amd as sce
    with pytest.raises(ValueError):
        sce.cross_entropy(torch.zeros(5), torch.zeros((), dtype=torch.int64))
    with pytest.raises(ValueError):
        sce.cross_entropy(torch.zeros(4, 5), torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError):
        sce.cross_entropy(torch.zeros(4, 5), torch.zeros(3, dtype=torch.int64))
    with pytest.raises((TypeError, ValueError)):
        sce.forward_raw(torch.zeros(4, 5, dtype=torch.float16).cuda() if torch.cuda.is_available()
                        else torch.zeros(4, 5, dtype=torch.float16), torch.zeros(4))


def test_shard_argument_checks():
    """The vocabulary-parallel entry points validate before touching memory."""
    f = FAKE
    assert _lib.ce_shard_partials(f, _lib.CE_F32, 4, 100, 100, 950, 1000, f, 0, -100, 0.0, 0.0, f,
                                  0) == _lib.CE_E_SHAPE  # v_offset + V > V_total
    assert _lib.ce_shard_partials(f, _lib.CE_F32, 4, 100, 100, -1, 1000, f, 0, -100, 0.0, 0.0, f,
                                  0) == _lib.CE_E_SHAPE
    assert _lib.ce_shard_partials(f, 9, 4, 100, 100, 0, 1000, f, 0, -100, 0.0, 0.0, f,
                                  0) == _lib.CE_E_DTYPE
    assert _lib.ce_shard_partials(0, _lib.CE_F32, 4, 100, 100, 0, 1000, f, 0, -100, 0.0, 0.0, f,
                                  0) == _lib.CE_E_NULL
    args = dict(logits=f, dtype=_lib.CE_F32, rows=4, V=100, row_stride=100, v_offset=0,
                V_total=1000, target=f, weight=0, ignore_index=-100, label_smoothing=0.0,
                lse_square_scale=0.0, softcap=0.0, reduction=_lib.CE_RED_SUM, flags=0,
                partials_all=f, num_shards=2, loss=f, z_loss=0, token_accuracy=0, argmax=0,
                counts=0, workspace=f, workspace_bytes=1 << 20, stream=0)
    assert _lib.ce_shard_finish(**dict(args, num_shards=0)) == _lib.CE_E_PARAM
    assert _lib.ce_shard_finish(**dict(args, label_smoothing=1.5)) == _lib.CE_E_PARAM
    assert _lib.ce_shard_finish(**dict(args, workspace_bytes=8)) == _lib.CE_E_WORKSPACE
    assert _lib.ce_shard_finish(**dict(args, workspace=f + 8)) == _lib.CE_E_WORKSPACE
    assert _lib.ce_shard_finish(**dict(args, loss=0)) == _lib.CE_E_NULL
    assert _lib.ce_shard_workspace_bytes(1000) >= 256 + 3 * 4000


def test_noalloc_rejects_problems_beyond_its_scratch():
    # host-side check before anything is enqueued: 62599 rows of fp32 at
    # V = 131072 need one layout step more than the static scratch holds
    for rows, want in ((62599, _lib.CE_E_SCRATCH), (1 << 20, _lib.CE_E_SCRATCH)):
        assert _lib.ce_workspace_bytes(rows, 131072, _lib.CE_F32, _lib.CE_F_GRAD) > \
            _lib.CE_FORWARD_NOALLOC_MAX_BYTES
        st = _lib.ce_forward_noalloc(1 << 20, _lib.CE_F32, rows, 131072, 131072, 1 << 20, 0,
                                     -100, 0.0, 0.0, 0.0, _lib.CE_RED_MEAN, _lib.CE_F_GRAD,
                                     1 << 20, 0, 0, 0, 0, 0, 0)
        assert st == want
    assert _lib.ce_workspace_bytes(62598, 131072, _lib.CE_F32, _lib.CE_F_GRAD) <= \
        _lib.CE_FORWARD_NOALLOC_MAX_BYTES
    # argument errors come first, as for ce_forward
    assert _lib.ce_forward_noalloc(1 << 20, 7, 4, 16, 16, 1 << 20, 0, -100, 0.0, 0.0, 0.0,
                                   _lib.CE_RED_MEAN, 0, 1 << 20, 0, 0, 0, 0, 0, 0) == \
        _lib.CE_E_DTYPE
    assert _lib.ce_forward_noalloc(1 << 20, _lib.CE_F32, 4, 16, 16, 1 << 20, 0, -100, 0.0, 0.0,
                                   0.0, _lib.CE_RED_MEAN, 0, 0, 0, 0, 0, 0, 0, 0) == \
        _lib.CE_E_NULL
