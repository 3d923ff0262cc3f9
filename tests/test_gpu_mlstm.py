"""GPU parity of the mLSTM kernel with exponential input gate and normaliser
(gla_mlstm_fwd) through the C ABI, against the fp64 mLSTM oracle (oracle.mlstm_recurrent,
pinned in test_oracle_mlstm.py) on the same seeded inputs.

Bar, as for the other forward paths: max |gpu - oracle| <= 1e-2 * RMS(oracle) for bf16 inputs
and <= 1e-4 * RMS(oracle) for fp32 inputs, over the whole output tensor.  The kernel returns
the stabilised state (C', n', m); exp(m) C' and exp(m) n' are compared with the oracle's
unstabilised C and n against their own RMS with the same factor.
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
    init = None if initial_state is None else tuple(cu(t) for t in initial_state)
    out, fin = gla.mlstm_fwd(cu(d["q"]), cu(d["k"]), cu(d["v"]), cu(d["log_f"]), cu(d["log_i"]),
                             initial_state=init, final_state=final_state)
    torch.cuda.synchronize()
    fin = None if fin is None else tuple(t.cpu() for t in fin)
    return out.cpu().double().numpy(), fin


def unstabilised(fin):
    C, n, m = (t.double().numpy() for t in fin)
    return C * np.exp(m)[..., None, None], n * np.exp(m)[..., None]


def run_oracle(d, initial_state=None):
    init = None
    if initial_state is not None:
        init = unstabilised(initial_state)
    return oracle.mlstm_recurrent(d["q"], d["k"], d["v"], d["log_f"], d["log_i"], init)


def check(w, got, ref, what):
    e = rel_err(got, ref)
    assert e <= TOL[w.dtype], "%s %s: max|err|/RMS = %.3e > %.0e" % (w.name, what, e, TOL[w.dtype])
    return e


def check_all(w, out, fin, ref):
    h, C, n = ref
    check(w, out, h, "out")
    if fin is not None:
        Cg, ng = unstabilised(fin)
        check(w, Cg, C, "final C")
        check(w, ng, n, "final n")


def rand_state(B, H, Dk, Dv, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, H, Dk, Dv, generator=g) * 0.3, torch.randn(B, H, Dk, generator=g) * 0.3,
            torch.randn(B, H, generator=g))


# bf16 with Dk = 256 and Dv a multiple of 128 runs the eight-wave kernel (128 value columns
# per workgroup), every other shape the four-wave one
SMALL = [("bf16", Dk, Dv) for Dk, Dv in ((64, 64), (128, 128), (64, 128), (256, 64), (128, 192), (256, 512),
                                          (256, 128), (256, 384))]
SMALL += [("f32", 64, Dv) for Dv in (64, 128)]


@pytest.mark.parametrize("dtype,Dk,Dv", SMALL)
@pytest.mark.parametrize("L", [1, 100, 333])
def test_mlstm_small_shapes(gpu_lib, dtype, Dk, Dv, L):
    w = gin.custom(2, 2, L, Dk, Dv, 64, dtype=dtype, gate="head", rule="mlstm")
    d = gin.make_inputs(w, seed=L + Dk)
    s0 = None if L == 100 else rand_state(2, 2, Dk, Dv, L)
    out, fin = run_gpu(gpu_lib, d, s0)
    check_all(w, out, fin, run_oracle(d, s0))


def _nonnegative_qk(d):
    # with q, k >= 0 every q_t . k_s is positive: no cancellation in q . n, and the read is a
    # weighted mean of the values wherever |q . n| >= 1, so its sensitivity to rounding stays
    # that of the arithmetic even when the gates span many orders of magnitude (with signed
    # q and k a normaliser that is a small difference of large terms magnifies any rounding
    # by |q| |n| / |q . n|, in fp64 as in fp32)
    d = dict(d)
    d["q"] = d["q"].abs()
    d["k"] = d["k"].abs()
    return d


@pytest.mark.parametrize("dtype,Dk,Dv", [("bf16", 64, 64), ("f32", 64, 64), ("bf16", 256, 128)])
@pytest.mark.parametrize("ig_std,offset", [(4.0, 0.0), (12.0, 0.0), (1.0, 100.0), (1.0, -60.0)])
def test_mlstm_extreme_input_gates(gpu_lib, dtype, Dk, Dv, ig_std, offset):
    # input gates spread over e^(+-3 ig_std), or all near e^100 (whose products overflow fp32
    # without the running maximum) or e^-60: every factor the kernel applies stays <= 1
    w = gin.custom(1, 2, 300, Dk, Dv, 64, dtype=dtype, gate="head", rule="mlstm", ig_std=ig_std)
    d = _nonnegative_qk(gin.make_inputs(w, seed=7))
    d["log_i"] = d["log_i"] + offset
    out, fin = run_gpu(gpu_lib, d)
    assert np.all(np.isfinite(out))
    h, C, n = run_oracle(d)
    check(w, out, h, "out")
    Cg, ng = unstabilised(fin)
    check(w, Cg, C, "final C")
    check(w, ng, n, "final n")


def test_mlstm_split_sequence_carries_the_state(gpu_lib):
    # the first part's stabilised final state, passed as the second part's initial state,
    # reproduces the whole-sequence run (and the oracle)
    w = gin.custom(2, 2, 400, 128, 128, 64, gate="head", rule="mlstm")
    d = gin.make_inputs(w, seed=11)
    whole, fin = run_gpu(gpu_lib, d)
    cut = 150
    first = {k: (v[:, :, :cut].contiguous() if k in ("q", "k", "v", "log_f", "log_i") else v) for k, v in d.items()}
    second = {k: (v[:, :, cut:].contiguous() if k in ("q", "k", "v", "log_f", "log_i") else v) for k, v in d.items()}
    o1, f1 = run_gpu(gpu_lib, first)
    o2, f2 = run_gpu(gpu_lib, second, initial_state=f1)
    ref = run_oracle(d)
    check_all(w, np.concatenate([o1, o2], axis=2), f2, ref)
    assert rel_err(np.concatenate([o1, o2], axis=2), whole) <= 1e-3


def test_mlstm_inactive_normaliser_matches_the_gated_linear_path(gpu_lib):
    # small queries keep |q . n| < 1: the output is q C, the sigmoid-free gated linear
    # recurrence with forget gate log_f and input gate log_i (gla_fwd_ex with a per-token gate)
    w = gin.custom(1, 2, 200, 64, 64, 64, gate="head", rule="mlstm")
    d = gin.make_inputs(w, seed=13)
    d["q"] = (d["q"].float() * 0.002).to(d["q"].dtype)
    out, fin = run_gpu(gpu_lib, d)
    h, C, n = run_oracle(d)
    qn = np.abs(np.einsum("bhtd,bhtd->bht", d["q"].double().numpy(), _running_n(d)))
    assert qn.max() < 1.0
    check_all(w, out, fin, (h, C, n))
    cu = lambda t: t.to("cuda").contiguous()
    lin, _ = gpu_lib.fwd(cu(d["q"]), cu(d["k"]), cu(d["v"]), cu(d["log_f"]), log_ig=cu(d["log_i"]), chunk=64)
    torch.cuda.synchronize()
    assert rel_err(out, lin.cpu().double().numpy()) <= 1e-2


def _running_n(d):
    k = d["k"].double().numpy()
    lf, li = d["log_f"].double().numpy(), d["log_i"].double().numpy()
    n = np.zeros(k.shape[:2] + (k.shape[-1],))
    res = np.zeros(k.shape)
    for t in range(k.shape[2]):
        n = np.exp(lf[:, :, t])[..., None] * n + np.exp(li[:, :, t])[..., None] * k[:, :, t]
        res[:, :, t] = n
    return res


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (256, 256)])
def test_mlstm_deterministic(gpu_lib, Dk, Dv):
    w = gin.custom(2, 3, 500, Dk, Dv, 64, gate="head", rule="mlstm")
    d = gin.make_inputs(w, seed=1)
    a, fa = run_gpu(gpu_lib, d)
    b, fb = run_gpu(gpu_lib, d)
    assert np.array_equal(a, b) and all(torch.equal(x, y) for x, y in zip(fa, fb))


@pytest.mark.parametrize("name", sorted(gin.MLSTM_WORKLOADS))
def test_mlstm_full_workload_whole_tensor(gpu_lib, name):
    # the mLSTM workload at full size, in the launch bench.py times, compared whole
    w = gin.MLSTM_WORKLOADS[name]
    d = gin.make_inputs(w, seed=0)
    print("mlstm workload %s" % name, flush=True)
    out, fin = run_gpu(gpu_lib, d)
    h, C, n = run_oracle(d)
    e = check(w, out, h, "out")
    Cg, ng = unstabilised(fin)
    ec = check(w, Cg, C, "final C")
    en = check(w, ng, n, "final n")
    print("  out max|err|/RMS = %.3e, final C %.3e, final n %.3e" % (e, ec, en), flush=True)


@pytest.mark.parametrize("dtype,B,H,L,Dk,Dv", [("bf16", 1, 2, 4096, 256, 512), ("bf16", 1, 1, 2048, 128, 128),
                                               ("f32", 1, 1, 3072, 64, 64), ("bf16", 2, 3, 2560, 64, 128)])
@pytest.mark.parametrize("with_s0", [False, True])
def test_mlstm_sequence_segments(gpu_lib, dtype, B, H, L, Dk, Dv, with_s0):
    # few (batch, head, value-slice) workgroups and a long sequence: the sequence runs as
    # segments (a pass from the zero state for every segment's own state, the join across
    # the segments, a pass from the entering states); outputs and final state against the oracle
    w = gin.custom(B, H, L, Dk, Dv, 64, dtype=dtype, gate="head", rule="mlstm")
    d = gin.make_inputs(w, seed=L + Dk)
    s0 = rand_state(B, H, Dk, Dv, seed=3) if with_s0 else None
    out, fin = run_gpu(gpu_lib, d, initial_state=s0)
    check_all(w, out, fin, run_oracle(d, s0))
