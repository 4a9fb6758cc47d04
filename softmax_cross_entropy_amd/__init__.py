"""MI355X-native fused softmax cross-entropy (forward + gradient-in-forward).

The compute path is hand-written HIP for gfx950 behind a C ABI
(include/ce.h, built into libce_mi355x.so); this package is its thin Python
binding. The library is loaded on first use and the call fails loudly if it
is missing -- there is no CPU or PyTorch fallback.
"""

from .functional import (CEOutput, CrossEntropyFunction, CrossEntropyLoss, backward_,
                         backward_recompute, cross_entropy, forward_raw, release_workspaces)
from .linear import (LinearCrossEntropyFunction, LinearCrossEntropyLoss, linear_cross_entropy,
                     linear_forward_raw)

__all__ = ["CEOutput", "CrossEntropyFunction", "CrossEntropyLoss", "backward_",
           "backward_recompute", "cross_entropy", "forward_raw", "release_workspaces",
           "LinearCrossEntropyFunction",
           "LinearCrossEntropyLoss", "linear_cross_entropy", "linear_forward_raw"]
