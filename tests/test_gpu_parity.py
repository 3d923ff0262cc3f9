"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar (written here, applied to every output element compared):
  bf16 inputs: max |gpu - oracle| <= 1e-2 * RMS(oracle)
  fp32 inputs: max |gpu - oracle| <= 1e-4 * RMS(oracle)
RMS is over the whole compared tensor (all batches, heads, tokens and columns, or all sampled
heads at full size); the final state is compared against its own RMS with the same factor.
Inputs come from the shared seeded generators; the oracle sees the same bytes.
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


def gate_name(w):
    return w.gate


def run_gpu(gla, d, w, chunk=None, seg_chunks=0, initial_state=None, final_state=True, tile_pairs=False):
    dev = "cuda"
    q, k, v = (d[x].to(dev) for x in "qkv")
    la = None if d["log_alpha"] is None else d["log_alpha"].to(dev)
    li = None if d["log_ig"] is None else d["log_ig"].to(dev)
    s0 = None if initial_state is None else initial_state.to(dev)
    out, fin = gla.fwd(q, k, v, la, log_ig=li, initial_state=s0, chunk=chunk or w.chunk,
                       final_state=final_state, seg_chunks=seg_chunks, tile_pairs=tile_pairs)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), None if fin is None else fin.cpu().double().numpy()


def run_oracle(d, w, initial_state=None, heads=None):
    sel = (lambda x: x) if heads is None else (lambda x: x if x is None else x.reshape(-1, *x.shape[2:])[heads][None])
    gate = w.gate
    la = d["log_alpha"]
    if heads is not None and gate == "head_const":
        H = w.H
        # [H] gate: pick each sampled head's value and present the heads as one batch row
        la = torch.stack([la[hh % H] for hh in heads])
        q, k, v = (sel(d[x]) for x in "qkv")
        return oracle.recurrent(q, k, v, "head_const", la, sel(d["log_ig"]), sel(initial_state))
    return oracle.recurrent(sel(d["q"]), sel(d["k"]), sel(d["v"]), gate, sel(la) if gate != "head_const" else la,
                            sel(d["log_ig"]), sel(initial_state))


def check(w, got, ref, what="out"):
    e = rel_err(got, ref)
    assert e <= TOL[w.dtype], "%s: %s max|err|/RMS = %.3e > %.0e" % (w.name, what, e, TOL[w.dtype])
    return e


# ------------------------------------------------------------------------------ small shapes
SMALL = []
for dtype in ("bf16", "f32"):
    for gate, ig in (("channel", False), ("none", False), ("head", True), ("head_const", False), ("channel", True)):
        for Dk, Dv in ((64, 64), (128, 128), (256, 64)):
            for chunk in (64, 128, 256, 512):
                SMALL.append((dtype, gate, ig, Dk, Dv, chunk))


def supported(gla, w, tile_pairs=False):
    """Status of the library's own support check for a workload (no GPU work)."""
    d = gin.make_inputs(w.with_(L=1), seed=0)
    t = {k: v for k, v in d.items()}
    out = torch.empty(w.B, w.H, 1, w.Dv)
    desc = gla.make_desc(t["q"], t["k"], t["v"], t["log_alpha"], t["log_ig"], None, out, None, w.chunk,
                         tile_pairs=tile_pairs)
    try:
        gla.workspace_size(desc)
        return True
    except gla.GlaError as e:
        assert e.status == gla.GLA_ERR_UNSUPPORTED
        return False


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv,chunk", SMALL)
@pytest.mark.parametrize("L", [1, 100, 333])
def test_small_shapes(gpu_lib, dtype, gate, ig, Dk, Dv, chunk, L):
    w = gin.custom(2, 2, L, Dk, Dv, chunk, dtype=dtype, gate=gate, input_gate=ig)
    assert supported(gpu_lib, w)
    d = gin.make_inputs(w, seed=L)
    out, fin = run_gpu(gpu_lib, d, w)
    ref, rfin = run_oracle(d, w)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv,chunk", [c for c in SMALL if c[5] > 64])
@pytest.mark.parametrize("L", [100, 333])
def test_small_shapes_tile_pairs(gpu_lib, dtype, gate, ig, Dk, Dv, chunk, L):
    # the tiled large-chunk form: terms between the 64-token tiles of a chunk as tile pairs
    w = gin.custom(2, 2, L, Dk, Dv, chunk, dtype=dtype, gate=gate, input_gate=ig)
    if not supported(gpu_lib, w, tile_pairs=True):
        # fp32 operands with several tiles per chunk: more LDS than a compute unit has
        assert dtype == "f32"
        pytest.skip("configuration reported unsupported (LDS budget)")
    d = gin.make_inputs(w, seed=L)
    out, fin = run_gpu(gpu_lib, d, w, tile_pairs=True)
    ref, rfin = run_oracle(d, w)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


@pytest.mark.parametrize("gate,ig,chunk", [("channel", False, 64), ("channel", True, 128), ("head", True, 256),
                                           ("head_const", False, 128), ("none", False, 64)])
@pytest.mark.parametrize("seg_chunks", [1, 2, 3])
@pytest.mark.parametrize("tile_pairs", [False, True])
def test_sequence_segments(gpu_lib, gate, ig, chunk, seg_chunks, tile_pairs):
    # several segments exercise the segment-state and segment-scan kernels; seg_chunks = 1 is
    # one state per chunk (the chunk-state / chunk-scan / chunk-output decomposition)
    w = gin.custom(1, 3, 1000, 128, 128, chunk, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=7)
    s0 = torch.randn(1, 3, 128, 128, generator=torch.Generator().manual_seed(3)) * 0.1
    out, fin = run_gpu(gpu_lib, d, w, seg_chunks=seg_chunks, initial_state=s0, tile_pairs=tile_pairs)
    ref, rfin = run_oracle(d, w, initial_state=s0)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


@pytest.mark.parametrize("gate,ig", [("head", True), ("head_const", False), ("none", False)])
@pytest.mark.parametrize("seg_chunks", [1, 3])
def test_sequence_segments_dk256(gpu_lib, gate, ig, seg_chunks):
    w = gin.custom(1, 2, 700, 256, 128, 64, gate=gate, input_gate=ig, scale_dim=256)
    d = gin.make_inputs(w, seed=8)
    s0 = torch.randn(1, 2, 256, 128, generator=torch.Generator().manual_seed(4)) * 0.05
    out, fin = run_gpu(gpu_lib, d, w, seg_chunks=seg_chunks, initial_state=s0)
    ref, rfin = run_oracle(d, w, initial_state=s0)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


def test_segment_modes_agree(gpu_lib):
    w = gin.custom(1, 2, 2048, 128, 128, 64, gate="channel")
    d = gin.make_inputs(w, seed=11)
    outs = [run_gpu(gpu_lib, d, w, seg_chunks=s)[0] for s in (1, 4, 32)]
    ref, _ = run_oracle(d, w)
    for o in outs:
        check(w, o, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,chunk", [("channel", 64), ("channel", 128), ("head", 64), ("head", 256)])
@pytest.mark.parametrize("tile_pairs", [False, True])
def test_gate_zero_keeps_only_current_token(gpu_lib, dtype, gate, chunk, tile_pairs):
    # alpha -> 0 (log gate -1e4 underflows to an exact zero): o_t = (q_t . k_t) v_t
    w = gin.custom(1, 2, 200, 64, 64, chunk, dtype=dtype, gate=gate)
    d = gin.make_inputs(w, seed=5)
    d["log_alpha"] = torch.full_like(d["log_alpha"], -1e4)
    if not supported(gpu_lib, w, tile_pairs):
        pytest.skip("configuration reported unsupported (LDS budget)")
    out, fin = run_gpu(gpu_lib, d, w, tile_pairs=tile_pairs)
    ref, rfin = run_oracle(d, w)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.3, 1.5, 6.0])
def test_strong_per_channel_decay(gpu_lib, dtype, scale):
    # large decay spans inside 16-token blocks take the exact diagonal path for some blocks
    w = gin.custom(1, 2, 257, 128, 64, 64, dtype=dtype, gate="channel")
    d = gin.make_inputs(w, seed=9)
    d["log_alpha"] = (d["log_alpha"] * 16.0 * scale).float()
    out, fin = run_gpu(gpu_lib, d, w)
    ref, rfin = run_oracle(d, w)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


def test_ungated_zero_gate_matches_no_gate(gpu_lib):
    w = gin.custom(1, 2, 300, 128, 128, 64, gate="channel")
    d = gin.make_inputs(w, seed=2)
    d0 = dict(d)
    d0["log_alpha"] = torch.zeros_like(d["log_alpha"])
    a, _ = run_gpu(gpu_lib, d0, w)
    wn = w.with_(gate="none")
    dn = dict(d)
    dn["log_alpha"] = None
    b, _ = run_gpu(gpu_lib, dn, wn)
    ref = oracle.bruteforce_ungated(d["q"][:, :, :40], d["k"][:, :, :40], d["v"][:, :, :40])
    check(w, a[:, :, :40], ref)
    check(w, b[:, :, :40], ref)


def test_deterministic(gpu_lib):
    w = gin.custom(2, 4, 777, 128, 128, 64, gate="channel", input_gate=True)
    d = gin.make_inputs(w, seed=1)
    a, fa = run_gpu(gpu_lib, d, w, seg_chunks=3)
    b, fb = run_gpu(gpu_lib, d, w, seg_chunks=3)
    assert np.array_equal(a, b) and np.array_equal(fa, fb)


def test_headline_entry_point_matches_general(gpu_lib):
    w = gin.custom(2, 2, 300, 128, 128, 64, gate="channel")
    d = gin.make_inputs(w, seed=4)
    q, k, v, la = (d[x].cuda() for x in ("q", "k", "v", "log_alpha"))
    out = torch.empty(2, 2, 300, 128, device="cuda")
    fin = torch.empty(2, 2, 128, 128, device="cuda")
    st = gpu_lib.fwd_headline(q, k, v, la, out, fin, chunk=64)
    assert st == 0
    o2, f2 = gpu_lib.fwd(q, k, v, la, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(fin, f2)
    # ungated through the headline entry point
    st = gpu_lib.fwd_headline(q, k, v, None, out, None, chunk=64)
    torch.cuda.synchronize()
    assert st == 0
    ref = oracle.bruteforce_ungated(d["q"][:, :, :32], d["k"][:, :, :32], d["v"][:, :, :32])
    check(w, out.cpu().double().numpy()[:, :, :32], ref)


def test_caller_workspace(gpu_lib):
    w = gin.custom(1, 2, 1500, 128, 128, 64, gate="channel")
    d = gin.make_inputs(w, seed=6)
    q, k, v, la = (d[x].cuda() for x in ("q", "k", "v", "log_alpha"))
    out = torch.empty(1, 2, 1500, 128, device="cuda")
    desc = gpu_lib.make_desc(q, k, v, la, out=out, chunk=64, seg_chunks=4)
    nbytes = gpu_lib.workspace_size(desc)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o1, f1 = gpu_lib.fwd(q, k, v, la, chunk=64, seg_chunks=4, workspace=ws)
    o2, f2 = gpu_lib.fwd(q, k, v, la, chunk=64, seg_chunks=4)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    small = torch.empty(nbytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.GlaError) as ei:
        gpu_lib.fwd(q, k, v, la, chunk=64, seg_chunks=4, workspace=small)
    assert ei.value.status == gpu_lib.GLA_ERR_WORKSPACE


# ------------------------------------------------------------------------------ full-size workloads
FULL = [
    ("ungated_f32_L256", None, False),
    ("gla_bf16_B8H16L2048", [0, 37, 127], False),
    ("retnet_bf16_B4H8L8192", [0, 7, 20, 31], False),
    ("retnet_bf16_B4H8L8192", [3, 30], True),
    ("long_gla_bf16_H16L32768_C64", [0, 9, 15], False),
    ("long_gla_bf16_H16L32768_C256", [0, 9, 15], False),
    ("long_gla_bf16_H16L32768_C256", [4], True),
    ("mlstm_sig_bf16_B8H8L8192", [0, 45], False),
    ("mlstm_sig_bf16_B8H8L8192", [63], True),
]


@pytest.mark.parametrize("name,heads,tile_pairs", FULL,
                         ids=[f[0] + ("_tile_pairs" if f[2] else "") for f in FULL])
def test_full_workload_sampled_heads(gpu_lib, name, heads, tile_pairs):
    w = gin.WORKLOADS[name]
    d = gin.make_inputs(w, seed=0)
    out, fin = run_gpu(gpu_lib, d, w, tile_pairs=tile_pairs)
    if heads is None:
        ref, rfin = run_oracle(d, w)
        check(w, out, ref)
        check(w, fin, rfin, "final_state")
        return
    ref, rfin = run_oracle(d, w, heads=heads)
    got = out.reshape(-1, *out.shape[2:])[heads][None]
    gfin = fin.reshape(-1, *fin.shape[2:])[heads][None]
    check(w, got, ref)
    check(w, gfin, rfin, "final_state")


# ------------------------------------------------------------------------------ recurrent step
def _token(d, w, t):
    """Inputs of token t: q, k [B,H,Dk], v [B,H,Dv], gate in the step layout, input gate [B,H]."""
    la = d["log_alpha"]
    if la is not None and w.gate in ("channel", "head"):
        la = la[:, :, t]
    li = None if d["log_ig"] is None else d["log_ig"][:, :, t]
    return d["q"][:, :, t], d["k"][:, :, t], d["v"][:, :, t], la, li


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,ig", [("channel", False), ("head", True), ("head_const", False), ("none", False),
                                     ("channel", True)])
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 192), (256, 64), (100, 64)])
def test_step_sequence_matches_recurrence(gpu_lib, dtype, gate, ig, Dk, Dv):
    # 9 steps from a random initial state against the fp64 recurrence over the same tokens
    w = gin.custom(2, 3, 9, Dk, Dv, 64, dtype=dtype, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=21)
    s0 = torch.randn(2, 3, Dk, Dv, generator=torch.Generator().manual_seed(5)) * 0.1
    state = s0.clone().cuda()
    outs = []
    for t in range(w.L):
        q, k, v, la, li = (None if x is None else x.cuda().contiguous() for x in _token(d, w, t))
        outs.append(gpu_lib.step(q, k, v, state, la, log_ig=li).cpu())
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=2).double().numpy()
    ref, rfin = run_oracle(d, w, initial_state=s0)
    check(w, got, ref)
    check(w, state.cpu().double().numpy(), rfin, "final_state")


@pytest.mark.parametrize("gate,ig,chunk", [("channel", False, 64), ("head", True, 256), ("head_const", False, 128)])
def test_step_continues_chunkwise_forward(gpu_lib, gate, ig, chunk):
    # chunkwise forward over L tokens, then recurrent steps for tokens L.. from its final state
    L, extra = 300, 5
    Dk = 256 if gate == "head" else 128
    w = gin.custom(2, 2, L + extra, Dk, 128, chunk, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=12)
    dl = dict(d)
    for key in ("q", "k", "v"):
        dl[key] = d[key][:, :, :L].contiguous()
    if gate in ("channel", "head"):
        dl["log_alpha"] = d["log_alpha"][:, :, :L].contiguous()
    if d["log_ig"] is not None:
        dl["log_ig"] = d["log_ig"][:, :, :L].contiguous()
    _, fin = run_gpu(gpu_lib, dl, w.with_(L=L))
    state = torch.from_numpy(fin).float().cuda()
    outs = []
    for t in range(L, L + extra):
        q, k, v, la, li = (None if x is None else x.cuda().contiguous() for x in _token(d, w, t))
        outs.append(gpu_lib.step(q, k, v, state, la, log_ig=li).cpu())
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=2).double().numpy()
    ref, rfin = run_oracle(d, w)
    check(w, got, ref[:, :, L:])
    check(w, state.cpu().double().numpy(), rfin, "final_state")
