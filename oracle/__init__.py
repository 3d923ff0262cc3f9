"""fp64 CPU oracle for the gated linear attention forward pass and its gradients (test
infrastructure only)."""
from .oracle import (GATE_KINDS, backward, build, bruteforce_ungated, chunkwise_form, expand_gate,  # noqa: F401
                     final_state_closed_form, load_library, parallel_form, recurrent, reduce_gate_grad,
                     threads)
