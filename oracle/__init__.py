"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .carve_oracle import carve_forward, carve_step, content_gate_bias, sigmoid  # noqa: F401
