"""fp64 CPU oracle for the gated linear attention forward pass, its gradients and the delta
rule (test infrastructure only)."""
from .oracle import (GATE_KINDS, backward, build, bruteforce_ungated, chunkwise_form, delta_chunkwise_form,  # noqa: F401
                     delta_gate, delta_recurrent, expand_gate, final_state_closed_form, load_library,
                     parallel_form, recurrent, reduce_gate_grad, threads)
