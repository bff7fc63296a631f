"""fp64 CPU oracle for the DoRA hot path -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and the CPU-baseline leg of bench.py may
import this package.  The product path (dora_adapter_factored_amd) never does.
"""
from .dora_oracle import (  # noqa: F401
    as_f64,
    adapted_weight_rows,
    dense_row_norm,
    factored_row_norm,
    magnitude_scale,
    compose_forward,
    compose_backward,
    compose_forward_inner,
    compose_backward_inner,
    dora_linear_forward,
    merged_weight,
    merge_with_scale,
)
