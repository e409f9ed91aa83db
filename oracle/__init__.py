"""Float64 CPU reference of the CARVE key-axis gated delta rule.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library's product path.
"""
from .carve_oracle import (forward, backward, backward_content, gates_from_logits,  # noqa: F401
                           forward_logits, backward_logits)
