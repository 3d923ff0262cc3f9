"""GPU parity of the delta-rule kernel (gla_delta_fwd, DeltaNet and Gated DeltaNet) through
the C ABI, against the fp64 delta-rule oracle (oracle.delta_recurrent, pinned in
test_oracle_delta.py) on the same seeded inputs.

Bar, as for the gated linear recurrence: max |gpu - oracle| <= 1e-2 * RMS(oracle) for bf16
inputs and <= 1e-4 * RMS(oracle) for fp32 inputs, over the whole output tensor; the final
state against its own RMS with the same factor.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_rnn_chunkwise_amd import inputs as gin

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def run_gpu(gla, d, initial_state=None, final_state=True):
    cu = lambda t: None if t is None else t.to("cuda").contiguous()
    out, fin = gla.delta_fwd(cu(d["q"]), cu(d["k"]), cu(d["v"]), cu(d["beta"]), cu(d["log_alpha"]),
                             initial_state=cu(initial_state), final_state=final_state)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), None if fin is None else fin.cpu().double().numpy()


def run_oracle(d, initial_state=None):
    return oracle.delta_recurrent(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], initial_state)


def check(w, got, ref, what):
    e = rel_err(got, ref)
    assert e <= TOL[w.dtype], "%s %s: max|err|/RMS = %.3e > %.0e" % (w.name, what, e, TOL[w.dtype])
    return e


SMALL = []
for Dk, Dv in ((64, 64), (128, 128), (64, 128), (256, 64), (128, 192)):
    for gate in ("none", "head", "head_const"):
        SMALL.append(("bf16", gate, Dk, Dv))
for Dv in (64, 128):
    for gate in ("none", "head", "head_const"):
        SMALL.append(("f32", gate, 64, Dv))


@pytest.mark.parametrize("dtype,gate,Dk,Dv", SMALL)
@pytest.mark.parametrize("L", [1, 100, 333])
def test_delta_small_shapes(gpu_lib, dtype, gate, Dk, Dv, L):
    w = gin.custom(2, 2, L, Dk, Dv, 64, dtype=dtype, gate=gate, rule="delta")
    d = gin.make_inputs(w, seed=L + Dk)
    s0 = None
    if L != 100:
        s0 = torch.randn(2, 2, Dk, Dv, generator=torch.Generator().manual_seed(L)) * 0.1
    out, fin = run_gpu(gpu_lib, d, s0)
    ref, rfin = run_oracle(d, s0)
    check(w, out, ref, "out")
    check(w, fin, rfin, "final_state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_delta_zero_gate_keeps_only_the_current_write(gpu_lib, dtype):
    # alpha = 0 (log gate -1e4): o_t = beta_t (q_t . k_t) v_t
    w = gin.custom(1, 2, 150, 64, 64, 64, dtype=dtype, gate="head", rule="delta")
    d = gin.make_inputs(w, seed=3)
    d["log_alpha"] = torch.full_like(d["log_alpha"], -1e4)
    out, fin = run_gpu(gpu_lib, d)
    ref, rfin = run_oracle(d)
    check(w, out, ref, "out")
    check(w, fin, rfin, "final_state")


def test_delta_zero_strength_keeps_the_state(gpu_lib):
    # beta = 0: the state only decays; o_t = g_t q_t S0
    w = gin.custom(1, 2, 130, 128, 128, 64, gate="head", rule="delta")
    d = gin.make_inputs(w, seed=4)
    d["beta"] = torch.zeros_like(d["beta"])
    s0 = torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(9)) * 0.1
    out, fin = run_gpu(gpu_lib, d, s0)
    ref, rfin = run_oracle(d, s0)
    check(w, out, ref, "out")
    check(w, fin, rfin, "final_state")


def test_delta_strength_one_on_repeated_keys(gpu_lib):
    # every token writes with beta = 1 and keys repeat within a chunk (the triangular system
    # has entries of size 1 below the diagonal): still the same map
    w = gin.custom(1, 2, 200, 64, 64, 64, gate="none", rule="delta")
    d = gin.make_inputs(w, seed=5)
    d["beta"] = torch.ones_like(d["beta"])
    k = d["k"].clone()
    k[:, :, 1::2] = k[:, :, 0::2][:, :, : k[:, :, 1::2].shape[2]]
    d["k"] = k
    out, fin = run_gpu(gpu_lib, d)
    ref, rfin = run_oracle(d)
    check(w, out, ref, "out")
    check(w, fin, rfin, "final_state")


def test_delta_deterministic(gpu_lib):
    w = gin.custom(2, 3, 500, 128, 128, 64, gate="head", rule="delta")
    d = gin.make_inputs(w, seed=1)
    a, fa = run_gpu(gpu_lib, d)
    b, fb = run_gpu(gpu_lib, d)
    assert np.array_equal(a, b) and np.array_equal(fa, fb)


@pytest.mark.parametrize("name", sorted(gin.DELTA_WORKLOADS))
def test_delta_full_workload_whole_tensor(gpu_lib, name):
    # the delta-rule workloads at full size, in the launch bench.py times, compared whole
    w = gin.DELTA_WORKLOADS[name]
    d = gin.make_inputs(w, seed=0)
    print("delta workload %s" % name, flush=True)
    out, fin = run_gpu(gpu_lib, d)
    ref, rfin = run_oracle(d)
    e = check(w, out, ref, "out")
    ef = check(w, fin, rfin, "final_state")
    print("  out max|err|/RMS = %.3e, final_state %.3e" % (e, ef), flush=True)
