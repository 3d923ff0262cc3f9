"""GPU parity of the backward pass (gla_bwd through the C ABI) against the fp64 oracle's
gradients (oracle.backward, itself pinned by finite differences).

Bar: every gradient satisfies max |gpu - oracle| <= 1e-4 * RMS(oracle) over the compared
tensor.  The backward's passes run with fp32 operands (bf16 inputs convert exactly), so the
fp32 rule applies to both input dtypes.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_rnn_chunkwise_amd import inputs as gin

pytestmark = pytest.mark.gpu

TOL = 1e-4


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def grads_in(w, seed, with_s0, with_df):
    g = torch.Generator().manual_seed(1000 + seed)
    dout = torch.randn(w.B, w.H, w.L, w.Dv, generator=g)
    s0 = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=g) * 0.1 if with_s0 else None
    df = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=g) * 0.1 if with_df else None
    return dout, s0, df


def run(gla, w, d, dout, s0, df):
    dev = "cuda"
    cu = lambda t: None if t is None else t.to(dev).contiguous()
    r = gla.bwd(cu(d["q"]), cu(d["k"]), cu(d["v"]), cu(dout), cu(d["log_alpha"]), log_ig=cu(d["log_ig"]),
                initial_state=cu(s0), dfinal_state=cu(df))
    torch.cuda.synchronize()
    return {k: None if v is None else v.cpu().double().numpy() for k, v in r.items()}


def check_all(got, ref, what):
    for key in ("dq", "dk", "dv", "dlog_alpha", "dlog_ig", "dinitial_state"):
        if ref[key] is None:
            assert got[key] is None, (what, key)
            continue
        e = rel_err(got[key], ref[key])
        assert e <= TOL, "%s %s: max|err|/RMS = %.3e" % (what, key, e)


CASES = []
for dtype in ("bf16", "f32"):
    for gate, ig in (("none", False), ("head", True), ("head", False), ("head_const", False)):
        for Dk, Dv in ((64, 64), (128, 128), (64, 128), (256, 64)):
            CASES.append((dtype, gate, ig, Dk, Dv))


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv", CASES)
@pytest.mark.parametrize("L", [1, 70, 333])
def test_backward_small_shapes(gpu_lib, dtype, gate, ig, Dk, Dv, L):
    w = gin.custom(2, 2, L, Dk, Dv, 64, dtype=dtype, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=L + Dk)
    dout, s0, df = grads_in(w, L, with_s0=(L != 70), with_df=(L != 333))
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, gate, d["log_alpha"], d["log_ig"], s0, df)
    check_all(got, ref, w.name)


def test_backward_strong_decay(gpu_lib):
    # per head and token gate near zero on some tokens: the reversed passes see the same decays
    w = gin.custom(1, 2, 150, 64, 64, 64, dtype="bf16", gate="head", input_gate=True)
    d = gin.make_inputs(w, seed=3)
    la = d["log_alpha"].clone()
    la[:, :, 40] = -30.0
    la[:, :, 100:103] = -1e4
    d["log_alpha"] = la
    dout, s0, df = grads_in(w, 5, True, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "head", la, d["log_ig"], s0, df)
    check_all(got, ref, "strong decay")


def test_backward_retnet_workload_sampled_heads(gpu_lib):
    # the RetNet workload at full size; (batch, head) slices are independent, so the oracle's
    # gradients of sampled slices are exact references for those slices of the full launch.
    # Head 5 is sampled in every batch so that its fixed-gate gradient (a sum over the batch
    # and the tokens) is checked too.
    w = gin.WORKLOADS["retnet_bf16_B4H8L8192"]
    d = gin.make_inputs(w, seed=0)
    dout, s0, df = grads_in(w, 0, False, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    H, hh = w.H, 5
    rows = [b * H + hh for b in range(w.B)]
    sel = lambda x: x.reshape(-1, *x.shape[2:])[rows][None]
    la = d["log_alpha"][hh].reshape(1, 1, 1).expand(1, len(rows), w.L).contiguous()
    ref = oracle.backward(sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(dout), "head", la, None, None, sel(df))
    for key in ("dq", "dk", "dv", "dinitial_state"):
        e = rel_err(got[key].reshape(-1, *got[key].shape[2:])[rows], ref[key][0])
        assert e <= TOL, "%s: max|err|/RMS = %.3e" % (key, e)
    total = float(ref["dlog_alpha"].sum())
    scale = max(abs(total), 1e-3 * float(np.abs(ref["dlog_alpha"]).sum()))
    assert abs(got["dlog_alpha"][hh] - total) <= TOL * scale, (got["dlog_alpha"][hh], total)


def test_backward_rejects_per_channel_gate(gpu_lib):
    w = gin.custom(1, 1, 64, 64, 64, 64, gate="channel")
    d = gin.make_inputs(w, seed=0)
    dout = torch.randn(1, 1, 64, 64)
    with pytest.raises(gpu_lib.GlaError) as ei:
        run(gpu_lib, w, d, dout, None, None)
    assert ei.value.status == gpu_lib.GLA_ERR_UNSUPPORTED
