"""GPU parity of the backward pass (gla_bwd through the C ABI) against the fp64 oracle's
gradients (oracle.backward, itself pinned by finite differences).

Bar, fp32 inputs (fp32 operands throughout): every gradient satisfies
max |gpu - oracle| <= 1e-4 * RMS(oracle) over the compared tensor, the forward pass's rule.

Bar, bf16 inputs: the passes take fp16 matrix operands (computed operands, states and the
output gradient scaled by a power of two, each rounded once to fp16, 2^-12 relative), so an
element's error scales with the magnitude of the terms that form it rather than with the
tensor's RMS (the rows of the first tokens, led by a large initial state, reach several
times the RMS, and an element of such a row may cancel to near zero).  Every element
satisfies |gpu - oracle| <= 1e-2 * max(RMS(oracle), scale_i), with scale_i the size of its
terms: for dq, dk, dv and dinitial_state the RMS of the element's row (last axis: one
state row and one gradient row form all of it); for dlog_ig_t = k_t . dk_t the product of
the norms; for the log-gate gradients, sums over tokens of q_t . dq_t - k_t . dk_t, the root
sum of squares of those norm products.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_rnn_chunkwise_amd import inputs as gin

pytestmark = pytest.mark.gpu

TOLS = {"f32": 1e-4, "bf16": 1e-2}


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


def dot_scale(a, b):
    """|a_t| |b_t| per token: the size of the terms of the dot product a_t . b_t."""
    a = np.asarray(a.double().numpy() if hasattr(a, "double") else a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.sqrt((a * a).sum(axis=-1) * (b * b).sum(axis=-1))


def row_scale(x):
    x = np.asarray(x, dtype=np.float64)
    return np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def gate_scale(d, ref, gate):
    """Root sum of squares of the dot products that each log-gate gradient element sums:
    per (b, h, t) over s >= t (per-token gate), per head over b and t weighted by t + 1
    (fixed gate, the sum over t of the per-token sums)."""
    if gate == "channel":
        # per channel the summed terms are the products q_s,d dq_s,d and k_s,d dk_s,d
        q = np.asarray(d["q"].double().numpy())
        k = np.asarray(d["k"].double().numpy())
        sq = (q * ref["dq"]) ** 2 + (k * ref["dk"]) ** 2
        return np.sqrt(np.cumsum(sq[:, :, ::-1], axis=2)[:, :, ::-1])
    sq = dot_scale(d["q"], ref["dq"]) ** 2 + dot_scale(d["k"], ref["dk"]) ** 2
    if gate == "head":
        return np.sqrt(np.cumsum(sq[..., ::-1], axis=-1)[..., ::-1])
    w = (np.arange(sq.shape[-1]) + 1.0) ** 2
    return np.sqrt((sq * w).sum(axis=(0, 2)))


def scaled_err(got, ref, scale):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.maximum(scale, rms), 1e-300)))


def check_all(got, ref, what, dtype, d=None, gate=None):
    tol = TOLS[dtype]
    for key in ("dq", "dk", "dv", "dlog_alpha", "dlog_ig", "dinitial_state"):
        if ref[key] is None:
            assert got[key] is None, (what, key)
            continue
        # the plain whole-tensor figure is logged beside the bar, so that the element-wise
        # scale of the bf16 bar cannot hide a change in the bulk of a tensor
        print("%s %s: max|err|/RMS = %.3e" % (what, key, rel_err(got[key], ref[key])), flush=True)
        if dtype == "f32":
            e = rel_err(got[key], ref[key])
        elif key == "dlog_alpha":
            e = scaled_err(got[key], ref[key], gate_scale(d, ref, gate))
        elif key == "dlog_ig":
            e = scaled_err(got[key], ref[key], dot_scale(d["k"], ref["dk"]))
        else:
            e = scaled_err(got[key], ref[key], row_scale(ref[key]))
        assert e <= tol, "%s %s: max|err|/scale = %.3e" % (what, key, e)


CASES = []
for dtype in ("bf16", "f32"):
    for gate, ig in (("none", False), ("head", True), ("head", False), ("head_const", False)):
        for Dk, Dv in ((64, 64), (128, 128), (64, 128), (256, 64), (64, 256), (256, 256)):
            CASES.append((dtype, gate, ig, Dk, Dv))


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv", CASES)
@pytest.mark.parametrize("L", [1, 70, 333])
def test_backward_small_shapes(gpu_lib, dtype, gate, ig, Dk, Dv, L):
    w = gin.custom(2, 2, L, Dk, Dv, 64, dtype=dtype, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=L + Dk)
    dout, s0, df = grads_in(w, L, with_s0=(L != 70), with_df=(L != 333))
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, gate, d["log_alpha"], d["log_ig"], s0, df)
    check_all(got, ref, w.name, dtype, d, gate)


SPLIT_CASES = []
for gate, ig in (("none", False), ("head", True), ("head", False), ("head_const", False)):
    for Dk in (64, 128, 256):
        SPLIT_CASES.append((gate, ig, Dk))


@pytest.mark.parametrize("gate,ig,Dk", SPLIT_CASES)
@pytest.mark.parametrize("L", [1, 70, 333])
def test_backward_dv512(gpu_lib, gate, ig, Dk, L):
    # Dv = 512 (the mLSTM head shape has Dk = 256): the dk and dq passes run over the two
    # 256-column halves of v and dout and add their outputs
    w = gin.custom(2, 2, L, Dk, 512, 64, dtype="bf16", gate=gate, input_gate=ig, scale_dim=256)
    d = gin.make_inputs(w, seed=L + Dk + 7)
    dout, s0, df = grads_in(w, L + 2, with_s0=(L != 70), with_df=(L != 333))
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, gate, d["log_alpha"], d["log_ig"], s0, df)
    check_all(got, ref, w.name, "bf16", d, gate)


def test_backward_mlstm_head_shape_long(gpu_lib):
    # the mLSTM workload's head shape and gates (Dk 256, Dv 512, per-token forget gate and
    # input gate) at length 4096 on four (batch, head) slices, every gradient compared whole
    w = gin.WORKLOADS["mlstm_sig_bf16_B8H8L8192"].with_(B=2, H=2, L=4096)
    d = gin.make_inputs(w, seed=3)
    dout, s0, df = grads_in(w, 3, True, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "head", d["log_alpha"], d["log_ig"], s0, df)
    check_all(got, ref, "mlstm head shape L4096", "bf16", d, "head")


@pytest.mark.parametrize("gate,ig,Dk,Dv", [("head", True, 128, 128), ("head_const", False, 128, 128),
                                            ("none", False, 64, 128), ("head", False, 256, 256)])
def test_backward_segmented_scalar_gate(gpu_lib, gate, ig, Dk, Dv):
    # two (batch, head) slices at length 34001: the passes split the sequence into dozens of
    # segments (segment-state kernels, scans, chunk-output workgroups starting from entry
    # states), ragged tail.  With Dk = Dv the dk pass takes the dv pass's segment-entry states,
    # read transposed; with Dk != Dv the two passes plan different segments and each forms its
    # own.  Initial state and final-state gradient given.
    w = gin.custom(1, 2, 34001, Dk, Dv, 64, dtype="bf16", gate=gate, input_gate=ig)
    for a, b in ((Dk, Dv), (Dv, Dk)):
        # the forward plan of each pass shape (planning only; the pointers are never used)
        pd = gpu_lib.GlaDesc()
        for key, val in dict(B=1, H=2, L=34001, Dk=a, Dv=b, chunk=64, in_dtype=gpu_lib.DTYPE_BF16,
                             gate_kind=gpu_lib.GATE_HEAD, q=256, k=256, v=256, log_alpha=256, out=256).items():
            setattr(pd, key, val)
        assert gpu_lib.plan(pd).n_seg > 8
    d = gin.make_inputs(w, seed=40 + Dk)
    dout, s0, df = grads_in(w, 41, True, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, gate, d["log_alpha"], d["log_ig"], s0, df)
    check_all(got, ref, "segmented %s Dk%d Dv%d" % (gate, Dk, Dv), "bf16", d, gate)


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
    check_all(got, ref, "strong decay", "bf16", d, "head")


def test_backward_retnet_workload_whole(gpu_lib):
    # the RetNet workload at full size (the launch bench.py --backward times), every gradient
    # compared whole against the oracle's, including the fixed gate's gradient per head (a sum
    # over the batch and the tokens)
    w = gin.WORKLOADS["retnet_bf16_B4H8L8192"]
    d = gin.make_inputs(w, seed=0)
    dout, s0, df = grads_in(w, 0, False, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "head_const", d["log_alpha"], None, None, df)
    check_all(got, ref, "retnet workload", "bf16", d, "head_const")


CH_CASES = []
for dtype in ("bf16", "f32"):
    for ig in (False, True):
        for Dk, Dv in ((64, 64), (128, 128), (64, 128), (256, 64), (128, 256), (256, 256)):
            CH_CASES.append((dtype, ig, Dk, Dv))


@pytest.mark.parametrize("dtype,ig,Dk,Dv", CH_CASES)
@pytest.mark.parametrize("L", [1, 70, 333])
def test_backward_per_channel_gate(gpu_lib, dtype, ig, Dk, Dv, L):
    # fp32 inputs: fp32 throughout, the fp32 bar; bf16 inputs run the dk and dq passes on fp16
    # operands (and the dv pass too for Dk <= 128), so the bf16 bar applies
    w = gin.custom(2, 2, L, Dk, Dv, 64, dtype=dtype, gate="channel", input_gate=ig)
    d = gin.make_inputs(w, seed=L + Dk + 3 * Dv)
    dout, s0, df = grads_in(w, L + 1, with_s0=(L != 70), with_df=(L != 333))
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "channel", d["log_alpha"], d["log_ig"], s0, df)
    check_all(got, ref, w.name, dtype, d, "channel")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_per_channel_block_decay_near_bound(gpu_lib, dtype):
    # channels whose decay over a 16-token block lands just above and just below 2^-8 (the
    # bound of the fp16 passes' factored form) and far below it
    w = gin.custom(1, 2, 200, 64, 128, 64, dtype=dtype, gate="channel", input_gate=True)
    d = gin.make_inputs(w, seed=12)
    la = d["log_alpha"].clone()
    la[:, :, :, :8] = -0.3    # 16 tokens: 2^-6.9
    la[:, :, :, 8:16] = -0.36  # 2^-8.3
    la[:, :, 60:140, 16:24] = -2.0
    d["log_alpha"] = la
    dout, s0, df = grads_in(w, 13, True, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "channel", la, d["log_ig"], s0, df)
    check_all(got, ref, "per-channel decay near the factor bound", dtype, d, "channel")


def test_backward_per_channel_strong_decay(gpu_lib):
    # channels with a near-zero or zero gate on some tokens, in the forward and reversed passes
    w = gin.custom(1, 2, 150, 64, 64, 64, dtype="bf16", gate="channel", input_gate=True)
    d = gin.make_inputs(w, seed=4)
    la = d["log_alpha"].clone()
    la[:, :, 40, :16] = -30.0
    la[:, :, 100:103, 8:40] = -1e4
    d["log_alpha"] = la
    dout, s0, df = grads_in(w, 6, True, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "channel", la, d["log_ig"], s0, df)
    check_all(got, ref, "per-channel strong decay", "bf16", d, "channel")


@pytest.mark.parametrize("ig", [False, True])
def test_backward_per_channel_many_segments(gpu_lib, ig):
    # few (batch, head) slices at length 2048: the value-gated passes split the sequence into
    # dozens of 64-token segments (state kernels, segment scans, and the log-gate gradient's
    # segment totals joined afterwards); initial state and final-state gradient given
    w = gin.custom(2, 2, 2048, 128, 128, 64, dtype="bf16", gate="channel", input_gate=ig)
    d = gin.make_inputs(w, seed=21 + ig)
    dout, s0, df = grads_in(w, 22, True, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "channel", d["log_alpha"], d["log_ig"], s0, df)
    check_all(got, ref, "per-channel, many segments", "bf16", d, "channel")


def test_backward_headline_workload_whole(gpu_lib):
    # the per-channel GLA workload at full size (the launch bench.py --backward times), every
    # gradient of every (batch, head) slice against the oracle's; every pass on fp16 operands,
    # so the bf16 bar applies
    w = gin.WORKLOADS["gla_bf16_B8H16L2048"]
    d = gin.make_inputs(w, seed=0)
    dout, s0, df = grads_in(w, 0, False, True)
    got = run(gpu_lib, w, d, dout, s0, df)
    ref = oracle.backward(d["q"], d["k"], d["v"], dout, "channel", d["log_alpha"], None, None, df)
    check_all(got, ref, "headline workload", "bf16", d, "channel")


@pytest.mark.parametrize("gate,ig", [("head", True), ("head_const", False), ("channel", True)])
def test_backward_bitwise_deterministic_and_caller_workspace(gpu_lib, gate, ig):
    # two calls with the library's own scratch and one with a caller workspace give the same
    # bits (no atomics decide an order anywhere in the backward)
    import ctypes
    w = gin.custom(2, 3, 777, 128, 128, 64, dtype="bf16", gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=11)
    dout, s0, df = grads_in(w, 11, True, True)
    a = run(gpu_lib, w, d, dout, s0, df)
    b = run(gpu_lib, w, d, dout, s0, df)
    cu = lambda t: None if t is None else t.to("cuda").contiguous()
    # every device tensor the descriptor points to stays referenced until the call has run
    q, k, v, la, li = cu(d["q"]), cu(d["k"]), cu(d["v"]), cu(d["log_alpha"]), cu(d["log_ig"])
    do_g, s0_g, df_g = cu(dout), cu(s0), cu(df)
    f = dict(dtype=torch.float32, device="cuda")
    out = {"dq": torch.empty(q.shape, **f), "dk": torch.empty(k.shape, **f), "dv": torch.empty(v.shape, **f),
           "dlog_alpha": torch.empty(la.shape, **f), "dlog_ig": torch.empty(li.shape, **f) if li is not None else None,
           "dinitial_state": torch.empty(2, 3, 128, 128, **f)}
    desc = gpu_lib.make_bwd_desc(q, k, v, do_g, out["dq"], out["dk"], out["dv"], la, li, s0_g, df_g,
                                 out["dlog_alpha"], out["dlog_ig"], out["dinitial_state"])
    lib = gpu_lib.load()
    need = ctypes.c_size_t(0)
    assert lib.gla_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(need)) == gpu_lib.GLA_OK
    ws = torch.full((need.value,), 0xFF, dtype=torch.uint8, device="cuda")  # stale contents must not matter
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), need.value
    st = torch.cuda.current_stream()
    assert lib.gla_bwd(ctypes.byref(desc), ctypes.c_void_p(st.cuda_stream)) == gpu_lib.GLA_OK
    torch.cuda.synchronize()
    c = {kk: None if vv is None else vv.cpu().double().numpy() for kk, vv in out.items()}
    for key in ("dq", "dk", "dv", "dlog_alpha", "dlog_ig", "dinitial_state"):
        if a[key] is None:
            continue
        assert np.array_equal(a[key], b[key]), key
        assert np.array_equal(a[key], c[key]), key
