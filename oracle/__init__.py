"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .carve_oracle import (carve_backward, carve_forward, carve_step, content_gate_bias,  # noqa: F401
                           decay_from_logits, l2_normalize, l2_normalize_backward, sigmoid)
