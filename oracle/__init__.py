"""fp64 CPU oracle for GDPA.  Test infrastructure only: used by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path."""
from .gdpa_oracle import (PHIS, as_f64, default_scale, gdpa_backward, gdpa_backward_bh,  # noqa: F401
                          gdpa_forward, gdpa_forward_bh, silu, silu_grad, sigmoid,
                          stacked_backward, stacked_forward, weight_generation,
                          weight_gradient)
