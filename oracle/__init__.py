"""fp64 CPU oracle for the gated linear attention forward pass, its gradients, the delta rule
and the mLSTM (test infrastructure only)."""
from .oracle import (GATE_KINDS, backward, build, bruteforce_ungated, chunkwise_form, delta_chunkwise_form,  # noqa: F401
                     delta_gate, delta_recurrent, expand_gate, final_state_closed_form, load_library,
                     mlstm_chunkwise_form, mlstm_parallel_form, mlstm_recurrent, mlstm_stabilized_recurrent,
                     parallel_form, recurrent, reduce_gate_grad, threads)
