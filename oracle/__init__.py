"""Float64 CPU oracle (test infrastructure only; see ce_oracle's header)."""
from .ce_oracle import (REDUCTIONS, OracleResult, RowResult, TargetSummary, ce_backward,
                        ce_forward, reduce_rows, rows_forward, summarize_targets, widen)
from .linear_oracle import (LinearResult, LinearRowsResult, grad_magnitudes, linear_forward,
                            linear_forward_rows)

__all__ = ["REDUCTIONS", "OracleResult", "RowResult", "TargetSummary", "ce_backward",
           "ce_forward", "reduce_rows", "rows_forward", "summarize_targets", "widen",
           "LinearResult", "LinearRowsResult", "grad_magnitudes", "linear_forward",
           "linear_forward_rows"]
