"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .carve_oracle import carve_forward, carve_step, content_gate_bias, decay_from_logits, sigmoid  # noqa: F401
