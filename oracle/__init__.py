"""Float64 CPU oracle (test infrastructure only; see oracle.py's header)."""
from .oracle import *  # noqa: F401,F403
from .oracle import (IGNORE_INDEX, LabelError, ForwardResult, BackwardResult,  # noqa: F401
                     supervised_rows, check_labels, logits, lse_two_pass, dense_forward,
                     dense_backward, dense_forward_backward, rows_forward, rows_grad_h,
                     tiled_forward_backward, reduce_rows, row_factors,
                     filtered_backward)
