"""ctypes binding of the C ABI in include/ce.h (argument marshalling only).

The functions here carry the same names as the C entry points and take the
same arguments: device pointers as Python ints, sizes, option values and a
raw hipStream_t. Every step of the computation runs in the HIP library;
there is no fallback: if the library is missing or fails to load, the call
raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch  # loads the process's HIP runtime first, so the library shares it

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libce_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

CE_OK = 0
CE_E_NULL = -1
CE_E_SHAPE = -2
CE_E_DTYPE = -3
CE_E_PARAM = -4
CE_E_WORKSPACE = -5
CE_E_HIP = -6
CE_E_TARGET_RANGE = -7
CE_E_EXCHANGE = -8
CE_E_SCRATCH = -9

# bytes of the static scratch ce_forward_noalloc holds per device
CE_FORWARD_NOALLOC_MAX_BYTES = 16 << 20

CE_F32 = 0
CE_BF16 = 1

CE_RED_NONE = 0
CE_RED_MEAN = 1
CE_RED_SUM = 2
REDUCTION_CODES = {"none": CE_RED_NONE, "mean": CE_RED_MEAN, "sum": CE_RED_SUM}

CE_F_GRAD = 1 << 0
CE_F_CHECK_TARGETS = 1 << 4
CE_F_FORCE_FUSED = 1 << 5
CE_F_FORCE_SPLITV = 1 << 6
CE_F_FORCE_SCALAR = 1 << 7
CE_F_SHAPE_ALT = 1 << 8
CE_F_EXCHANGE_ONE_POLL = 1 << 9
CE_F_LINEAR_ON_CHIP = 1 << 10

CE_PATH_FUSED = 1
CE_PATH_SPLITV = 2
CE_PATH_SCALAR = 3
PATH_NAMES = {CE_PATH_FUSED: "fused", CE_PATH_SPLITV: "splitv", CE_PATH_SCALAR: "scalar"}

# Every symbol include/ce.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGNATURES = {
    "ce_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, ctypes.c_int, ctypes.c_uint32]),
    "ce_plan_path": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_float,
                                    ctypes.c_uint32]),
    "ce_forward": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _I64,
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                  ctypes.c_uint32, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                  _P]),
    "ce_forward_noalloc": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _I64,
                                          ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_int, ctypes.c_uint32, _P, _P, _P, _P, _P, _P,
                                          _P]),
    "ce_backward": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_int, _P]),
    "ce_backward_recompute": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _I64,
                                             ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                             ctypes.c_int, _P, _P, ctypes.c_int, _P, _I64, _P,
                                             ctypes.c_size_t, _P]),
    "ce_linear_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, ctypes.c_uint32]),
    "ce_linear_forward": (ctypes.c_int, [_P, _I64, _P, _I64, ctypes.c_int, _I64, _I64, _I64,
                                         _P, _P, _I64, ctypes.c_float, ctypes.c_float,
                                         ctypes.c_float, ctypes.c_int, ctypes.c_uint32, _P,
                                         ctypes.c_int, _I64, _P, _P, _P, _P, _P, _P, _I64, _P,
                                         _I64, _P, ctypes.c_size_t, _P]),
    "ce_shard_workspace_bytes": (ctypes.c_size_t, [_I64]),
    "ce_shard_partials": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _P, _P,
                                         _I64, ctypes.c_float, ctypes.c_float, _P, _P]),
    "ce_shard_finish": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _P, _P,
                                       _I64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_int, ctypes.c_uint32, _P, ctypes.c_int, _P, _P,
                                       _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "ce_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    # include/ce_stream.h: the measurement stream kernels
    "ce_stream_num_configs": (ctypes.c_int, []),
    "ce_stream_config": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_int)]),
    "ce_stream_resident": (_I64, [ctypes.c_int, ctypes.c_int]),
    "ce_stream_run": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_size_t, _I64,
                                     _P, _P]),
}
SYMBOLS = tuple(_SIGNATURES)

_lock = threading.Lock()
_handle = None


class CEError(RuntimeError):
    """A non-zero ce_status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ce_status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if it has not been built."""
    global _handle
    if _handle is not None:
        return _handle
    with _lock:
        if _handle is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_NAME} is not built (expected at {LIB_PATH}); build it with "
                    "`python -m softmax_cross_entropy_amd.build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _handle = h
    return _handle


def ce_status_string(status: int) -> str:
    return lib().ce_status_string(int(status)).decode()


def ce_workspace_bytes(rows: int, V: int, dtype: int, flags: int) -> int:
    return int(lib().ce_workspace_bytes(rows, V, dtype, flags))


def ce_plan_path(logits: int, dtype: int, rows: int, V: int, row_stride: int, weight: int,
                 label_smoothing: float, flags: int) -> int:
    return int(lib().ce_plan_path(logits, dtype, rows, V, row_stride, weight,
                                  label_smoothing, flags))


def ce_forward(logits: int, dtype: int, rows: int, V: int, row_stride: int, target: int,
               weight: int, ignore_index: int, label_smoothing: float, lse_square_scale: float,
               softcap: float, reduction: int, flags: int, loss: int, z_loss: int,
               token_accuracy: int, argmax: int, counts: int, row_stats: int, workspace: int,
               workspace_bytes: int, stream: int) -> int:
    """Raw call; returns the ce_status (0 = CE_OK)."""
    return int(lib().ce_forward(logits, dtype, rows, V, row_stride, target, weight,
                                ignore_index, label_smoothing, lse_square_scale, softcap,
                                reduction, flags, loss, z_loss, token_accuracy, argmax, counts,
                                row_stats, workspace, workspace_bytes, stream))


def ce_forward_noalloc(logits: int, dtype: int, rows: int, V: int, row_stride: int,
                       target: int, weight: int, ignore_index: int, label_smoothing: float,
                       lse_square_scale: float, softcap: float, reduction: int, flags: int,
                       loss: int, z_loss: int, token_accuracy: int, argmax: int, counts: int,
                       row_stats: int, stream: int) -> int:
    """Raw call; returns the ce_status (0 = CE_OK)."""
    return int(lib().ce_forward_noalloc(logits, dtype, rows, V, row_stride, target, weight,
                                        ignore_index, label_smoothing, lse_square_scale,
                                        softcap, reduction, flags, loss, z_loss, token_accuracy,
                                        argmax, counts, row_stats, stream))


def ce_backward_recompute(logits: int, dtype: int, rows: int, V: int, row_stride: int,
                          target: int, weight: int, ignore_index: int, label_smoothing: float,
                          lse_square_scale: float, softcap: float, reduction: int,
                          row_stats: int, grad_output: int, per_row: int, grad: int,
                          grad_stride: int, workspace: int, workspace_bytes: int,
                          stream: int) -> int:
    """Raw call; returns the ce_status (0 = CE_OK)."""
    return int(lib().ce_backward_recompute(logits, dtype, rows, V, row_stride, target, weight,
                                           ignore_index, label_smoothing, lse_square_scale,
                                           softcap, reduction, row_stats, grad_output, per_row,
                                           grad, grad_stride, workspace, workspace_bytes,
                                           stream))


def ce_backward(grad: int, dtype: int, rows: int, V: int, row_stride: int, grad_output: int,
                per_row: int, stream: int) -> int:
    """Raw call; returns the ce_status (0 = CE_OK)."""
    return int(lib().ce_backward(grad, dtype, rows, V, row_stride, grad_output, per_row, stream))


def ce_linear_workspace_bytes(rows: int, H: int, V: int, chunk_rows: int, flags: int) -> int:
    return int(lib().ce_linear_workspace_bytes(rows, H, V, chunk_rows, flags))


def ce_linear_forward(hidden: int, ld_hidden: int, weight: int, ld_weight: int, dtype: int,
                      rows: int, H: int, V: int, target: int, class_weight: int,
                      ignore_index: int, label_smoothing: float, lse_square_scale: float,
                      softcap: float, reduction: int, flags: int, grad_output: int,
                      per_row: int, chunk_rows: int, loss: int, z_loss: int,
                      token_accuracy: int, argmax: int, counts: int, grad_hidden: int,
                      ld_grad_hidden: int, grad_weight: int, ld_grad_weight: int,
                      workspace: int, workspace_bytes: int, stream: int) -> int:
    """Raw call; returns the ce_status (0 = CE_OK)."""
    return int(lib().ce_linear_forward(hidden, ld_hidden, weight, ld_weight, dtype, rows, H, V,
                                       target, class_weight, ignore_index, label_smoothing,
                                       lse_square_scale, softcap, reduction, flags, grad_output,
                                       per_row, chunk_rows, loss, z_loss, token_accuracy, argmax,
                                       counts, grad_hidden, ld_grad_hidden, grad_weight,
                                       ld_grad_weight, workspace, workspace_bytes, stream))


def ce_shard_workspace_bytes(rows: int) -> int:
    return int(lib().ce_shard_workspace_bytes(rows))


def ce_shard_partials(logits: int, dtype: int, rows: int, V: int, row_stride: int, v_offset: int,
                      V_total: int, target: int, weight: int, ignore_index: int,
                      label_smoothing: float, softcap: float, partials: int, stream: int) -> int:
    """Raw call; returns the ce_status (0 = CE_OK)."""
    return int(lib().ce_shard_partials(logits, dtype, rows, V, row_stride, v_offset, V_total,
                                       target, weight, ignore_index, label_smoothing, softcap,
                                       partials, stream))


def ce_shard_finish(logits: int, dtype: int, rows: int, V: int, row_stride: int, v_offset: int,
                    V_total: int, target: int, weight: int, ignore_index: int,
                    label_smoothing: float, lse_square_scale: float, softcap: float,
                    reduction: int, flags: int, partials_all: int, num_shards: int, loss: int,
                    z_loss: int, token_accuracy: int, argmax: int, counts: int, workspace: int,
                    workspace_bytes: int, stream: int) -> int:
    """Raw call; returns the ce_status (0 = CE_OK)."""
    return int(lib().ce_shard_finish(logits, dtype, rows, V, row_stride, v_offset, V_total,
                                     target, weight, ignore_index, label_smoothing,
                                     lse_square_scale, softcap, reduction, flags, partials_all,
                                     num_shards, loss, z_loss, token_accuracy, argmax, counts,
                                     workspace, workspace_bytes, stream))


CE_STREAM_READ = 0
CE_STREAM_WRITE = 1
CE_STREAM_INPLACE = 2
CE_STREAM_COPY = 3
CE_STREAM_FLUSH = 4


def ce_stream_num_configs() -> int:
    return int(lib().ce_stream_num_configs())


def ce_stream_config(config: int):
    """(block, nreg) of a stream-kernel chunk shape."""
    b, n = ctypes.c_int(0), ctypes.c_int(0)
    check(lib().ce_stream_config(config, ctypes.byref(b), ctypes.byref(n)), "ce_stream_config")
    return b.value, n.value


def ce_stream_resident(kind: int, config: int) -> int:
    return int(lib().ce_stream_resident(kind, config))


def ce_stream_run(kind: int, config: int, dst: int, src: int, nbytes: int, grid: int,
                  sink: int, stream: int) -> int:
    """Raw call; returns the status (0 = CE_OK)."""
    return int(lib().ce_stream_run(kind, config, dst, src, nbytes, grid, sink, stream))


def check(status: int, where: str) -> None:
    if status != CE_OK:
        raise CEError(status, where)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return CE_F32
    if dt == torch.bfloat16:
        return CE_BF16
    raise TypeError(f"logits dtype must be float32 or bfloat16, got {dt}")
