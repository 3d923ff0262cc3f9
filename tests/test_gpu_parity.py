"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar (written here, applied to every output element compared):
  bf16 inputs: max |gpu - oracle| <= 1e-2 * RMS(oracle)
  fp32 inputs: max |gpu - oracle| <= 1e-4 * RMS(oracle)
RMS is over the whole compared tensor (all batches, heads, tokens and columns, also at the
full workload sizes); the final state is compared against its own RMS with the same factor.
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


def run_gpu(gla, d, w, chunk=None, seg_chunks=0, initial_state=None, final_state=True, tile_pairs=False,
            query_tiles=False):
    dev = "cuda"
    q, k, v = (d[x].to(dev) for x in "qkv")
    la = None if d["log_alpha"] is None else d["log_alpha"].to(dev)
    li = None if d["log_ig"] is None else d["log_ig"].to(dev)
    s0 = None if initial_state is None else initial_state.to(dev)
    out, fin = gla.fwd(q, k, v, la, log_ig=li, initial_state=s0, chunk=chunk or w.chunk,
                       final_state=final_state, seg_chunks=seg_chunks, tile_pairs=tile_pairs,
                       query_tiles=query_tiles)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), None if fin is None else fin.cpu().double().numpy()


def run_oracle(d, w, initial_state=None):
    return oracle.recurrent(d["q"], d["k"], d["v"], w.gate, d["log_alpha"], d["log_ig"], initial_state)


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


def supported(gla, w, tile_pairs=False, query_tiles=False):
    """Status of the library's own support check for a workload (no GPU work)."""
    d = gin.make_inputs(w.with_(L=1), seed=0)
    t = {k: v for k, v in d.items()}
    out = torch.empty(w.B, w.H, 1, w.Dv)
    desc = gla.make_desc(t["q"], t["k"], t["v"], t["log_alpha"], t["log_ig"], None, out, None, w.chunk,
                         tile_pairs=tile_pairs, query_tiles=query_tiles)
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


@pytest.mark.parametrize("dtype,gate,ig", [("bf16", "channel", False), ("bf16", "head", True), ("f32", "none", False),
                                          ("f32", "channel", True)])
@pytest.mark.parametrize("chunk", [16, 32])
def test_small_chunk_sizes(gpu_lib, dtype, gate, ig, chunk):
    # chunks of 16 and 32 tokens (run as 64-token tiles) against the oracle, ragged tail
    w = gin.custom(2, 2, 333, 128 if dtype == "bf16" else 64, 128, chunk, dtype=dtype, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=chunk)
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


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv,chunk", SMALL)
@pytest.mark.parametrize("L", [100, 333])
def test_small_shapes_query_tiles(gpu_lib, dtype, gate, ig, Dk, Dv, chunk, L):
    # the tiled large-chunk form with one workgroup per query tile of a chunk, every chunk its
    # own segment (chunk-start states from the segment-state kernel and scan); ragged tails
    # leave the last chunk with fewer tiles than the others
    w = gin.custom(2, 2, L, Dk, Dv, chunk, dtype=dtype, gate=gate, input_gate=ig)
    if not supported(gpu_lib, w, query_tiles=True):
        assert dtype == "f32" and chunk > 64
        pytest.skip("configuration reported unsupported (LDS budget)")
    d = gin.make_inputs(w, seed=L + 1)
    out, fin = run_gpu(gpu_lib, d, w, query_tiles=True)
    ref, rfin = run_oracle(d, w)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


@pytest.mark.parametrize("gate,ig,chunk,L", [("channel", True, 256, 1000), ("head", True, 512, 1200),
                                             ("head_const", False, 128, 777), ("none", False, 256, 64 * 12)])
def test_query_tiles_initial_state(gpu_lib, gate, ig, chunk, L):
    # chunk-start states built on a given initial state; the final state comes from the
    # workgroup of the last tile of the last chunk
    w = gin.custom(1, 3, L, 128, 128, chunk, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=11)
    s0 = torch.randn(1, 3, 128, 128, generator=torch.Generator().manual_seed(5)) * 0.1
    out, fin = run_gpu(gpu_lib, d, w, initial_state=s0, query_tiles=True)
    ref, rfin = run_oracle(d, w, initial_state=s0)
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


# ------------------------------------------------------------------------------ padded shapes
# Dk and Dv multiples of 16 that the kernels do not take directly run on zero-padded copies
# (Dk to 64, 128 or 256; Dv to the next multiple of 64)
PADDED = [("bf16", "channel", False, 96, 128), ("bf16", "channel", True, 32, 48), ("bf16", "head", True, 160, 80),
          ("bf16", "head_const", False, 208, 144), ("bf16", "none", False, 16, 16), ("f32", "channel", True, 48, 112),
          ("f32", "head", False, 96, 64), ("bf16", "channel", False, 240, 272)]


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv", PADDED)
@pytest.mark.parametrize("chunk", [64, 128])
def test_padded_shapes(gpu_lib, dtype, gate, ig, Dk, Dv, chunk):
    w = gin.custom(2, 2, 333, Dk, Dv, chunk, dtype=dtype, gate=gate, input_gate=ig)
    d = gin.make_inputs(w, seed=Dk + Dv)
    s0 = torch.randn(2, 2, Dk, Dv, generator=torch.Generator().manual_seed(Dk)) * 0.1
    out, fin = run_gpu(gpu_lib, d, w, initial_state=s0)
    ref, rfin = run_oracle(d, w, initial_state=s0)
    check(w, out, ref)
    check(w, fin, rfin, "final_state")


def test_padded_shape_entry_points(gpu_lib):
    # the 13-argument entry point and the allocation-free one take the padded shapes too
    w = gin.custom(1, 2, 200, 96, 80, 64, gate="channel")
    d = gin.make_inputs(w, seed=5)
    ref, rfin = run_oracle(d, w)
    dev = "cuda"
    q, k, v, la = (d[x].to(dev) for x in ("q", "k", "v", "log_alpha"))
    out = torch.empty(1, 2, 200, 80, device=dev)
    fin = torch.empty(1, 2, 96, 80, device=dev)
    assert gpu_lib.fwd_headline(q, k, v, la, out, fin, chunk=64) == gpu_lib.GLA_OK
    torch.cuda.synchronize()
    check(w, out.cpu().double().numpy(), ref)
    check(w, fin.cpu().double().numpy(), rfin, "final_state")
    out2, fin2 = gpu_lib.fwd_noalloc(q, k, v, la, chunk=64, final_state=torch.empty_like(fin))
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(fin2, fin)


# ------------------------------------------------------------------------------ full-size workloads
# Every full-size workload in the launch configuration bench.py times, compared whole: every
# (batch, head) slice of the output and of the final state, with RMS over the whole tensor.
FULL = [
    ("ungated_f32_L256", ""),
    ("gla_bf16_B8H16L2048", ""),
    ("retnet_bf16_B4H8L8192", ""),
    ("retnet_bf16_B4H8L8192", "tile_pairs"),
    ("retnet_bf16_B4H8L8192", "query_tiles"),
    ("long_gla_bf16_H16L32768_C64", ""),
    ("long_gla_bf16_H16L32768_C256", ""),
    ("long_gla_bf16_H16L32768_C256", "tile_pairs"),
    ("long_gla_bf16_H16L32768_C256", "query_tiles"),
    ("mlstm_sig_bf16_B8H8L8192", ""),
    ("mlstm_sig_bf16_B8H8L8192", "tile_pairs"),
    ("mlstm_sig_bf16_B8H8L8192", "query_tiles"),
]
_FULL_REF = {}


def full_reference(w, d):
    """The oracle over the whole workload, kept for the workload's other launch forms (the
    C64 and C256 long-sequence workloads draw the same inputs)."""
    key = (w.B, w.H, w.L, w.Dk, w.Dv, w.dtype, w.gate, w.input_gate, d["sha256"])
    if key not in _FULL_REF:
        _FULL_REF.clear()
        _FULL_REF[key] = run_oracle(d, w)
    return _FULL_REF[key]


@pytest.mark.parametrize("name,form", FULL, ids=[f[0] + ("_" + f[1] if f[1] else "") for f in FULL])
def test_full_workload_whole_tensor(gpu_lib, name, form):
    w = gin.WORKLOADS[name]
    d = gin.make_inputs(w, seed=0)
    print("full workload %s %s" % (name, form or "default"), flush=True)
    out, fin = run_gpu(gpu_lib, d, w, tile_pairs=form == "tile_pairs", query_tiles=form == "query_tiles")
    ref, rfin = full_reference(w, d)
    e = check(w, out, ref)
    ef = check(w, fin, rfin, "final_state")
    print("  out max|err|/RMS = %.3e, final_state %.3e" % (e, ef), flush=True)


# ------------------------------------------------------------------------------ longest slices
# The longest sequence a (batch, head) slice may have: one slice is addressed with 32-bit byte
# offsets, (L + 1024) * max(Dk, Dv) * 4 < 2^32.  Too long for the oracle's whole recurrence,
# so the comparison uses a property that holds at any length: a token whose log gate is -1e4 on
# every channel (a decay of exactly zero in fp32) starts the state afresh, S_t = i_t k_t^T v_t,
# so the outputs from that token on, and the final state after the last such token, equal the
# recurrence run from zero over the tokens from it alone.  Several such tokens are planted (one
# at the start, one in the middle, one near the end) and the window after each is compared
# whole with the oracle.  Two slices, so the second slice's fp32 gate and output rows start
# past 4 GiB (slice bases are 64-bit addresses).  Inputs are seeded draws made on the device.
LONGEST = [
    # dtype, gate, input gate, Dk, Dv
    ("bf16", "channel", False, 128, 128),
    ("bf16", "head", True, 256, 512),
]


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv", LONGEST)
def test_longest_slice_windows(gpu_lib, dtype, gate, ig, Dk, Dv):
    B, H = 1, 2
    L = (1 << 32) // (max(Dk, Dv) * 4) - 1025
    assert (L + 1024) * max(Dk, Dv) * 4 < (1 << 32) <= (L + 1025) * max(Dk, Dv) * 4
    dev = "cuda"
    print("longest slice %s %s Dk%d Dv%d L=%d" % (dtype, gate, Dk, Dv, L), flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(77 + Dk)
    wdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = (torch.randn(B, H, L, Dk, generator=g, device=dev) / Dk ** 0.5).to(wdt)
    k = (torch.randn(B, H, L, Dk, generator=g, device=dev) / Dk ** 0.5).to(wdt)
    v = (torch.randn(B, H, L, Dv, generator=g, device=dev) / Dk ** 0.5).to(wdt)
    shape = (B, H, L, Dk) if gate == "channel" else (B, H, L)
    la = torch.nn.functional.logsigmoid(torch.randn(*shape, generator=g, device=dev)) / 16
    li = torch.nn.functional.logsigmoid(torch.randn(B, H, L, generator=g, device=dev)) if ig else None
    W = 1000
    starts = [0, L // 3 + 17, L - 1500]
    for t in starts:
        la[:, :, t] = -1e4
    out, fin = gpu_lib.fwd(q, k, v, la, log_ig=li, chunk=64)
    torch.cuda.synchronize()
    cpu = lambda x, a, b: None if x is None else x[:, :, a:b].cpu()
    for t in starts:
        e = min(L, t + W) if t != starts[-1] else L
        ref, rfin = oracle.recurrent(cpu(q, t, e), cpu(k, t, e), cpu(v, t, e), gate, cpu(la, t, e), cpu(li, t, e))
        got = out[:, :, t:e].cpu().double().numpy()
        err = rel_err(got, ref)
        print("  window [%d, %d): out max|err|/RMS = %.3e" % (t, e, err), flush=True)
        assert err <= TOL[dtype], "window at %d: %.3e" % (t, err)
        if e == L:
            ef = rel_err(fin.cpu().double().numpy(), rfin)
            print("  final_state max|err|/RMS = %.3e" % ef, flush=True)
            assert ef <= TOL[dtype]
    del q, k, v, la, li, out, fin
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,gate,ig,Dk,Dv", LONGEST)
def test_longest_slice_state_across_segments(gpu_lib, dtype, gate, ig, Dk, Dv):
    # The state carried across the whole longest slice (dozens of sequence segments, the
    # segment-state kernel and the scan): every log gate is 0 (no decay) and every key is zero
    # except at 64 planted tokens spread over the sequence, so the state at token t is the
    # input-gated sum of the planted tokens' k^T v up to t, exactly the recurrence over the
    # planted tokens alone.  A window's outputs are compared with the recurrence run over the
    # planted tokens before it followed by the window's own tokens; the last window also
    # compares the final state.
    B, H = 1, 2
    L = (1 << 32) // (max(Dk, Dv) * 4) - 1025
    dev = "cuda"
    print("longest slice, state across segments: %s %s Dk%d Dv%d L=%d" % (dtype, gate, Dk, Dv, L), flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(91 + Dk)
    wdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = (torch.randn(B, H, L, Dk, generator=g, device=dev) / Dk ** 0.5).to(wdt)
    v = (torch.randn(B, H, L, Dv, generator=g, device=dev) / Dk ** 0.5).to(wdt)
    rng = np.random.default_rng(5 + Dk)
    planted = np.sort(rng.choice(L - 2000, size=64, replace=False))
    k = torch.zeros(B, H, L, Dk, dtype=wdt, device=dev)
    kp = torch.randn(B, H, len(planted), Dk, generator=g, device=dev) / Dk ** 0.5
    k[:, :, torch.from_numpy(planted).to(dev)] = kp.to(wdt)
    shape = (B, H, L, Dk) if gate == "channel" else (B, H, L)
    la = torch.zeros(*shape, device=dev)
    li = torch.nn.functional.logsigmoid(torch.randn(B, H, L, generator=g, device=dev)) if ig else None
    out, fin = gpu_lib.fwd(q, k, v, la, log_ig=li, chunk=64)
    torch.cuda.synchronize()
    W = 1000
    for a in (L // 2 + 5, L - 1200):
        b = min(L, a + W) if a != L - 1200 else L
        idx = torch.from_numpy(np.concatenate([planted[planted < a], np.arange(a, b)])).to(dev)
        sel = lambda x: None if x is None else x[:, :, idx].cpu()
        ref, rfin = oracle.recurrent(sel(q), sel(k), sel(v), gate, sel(la), sel(li))
        n = b - a
        got = out[:, :, a:b].cpu().double().numpy()
        err = rel_err(got, ref[:, :, -n:])
        print("  window [%d, %d) after %d planted tokens: out max|err|/RMS = %.3e"
              % (a, b, int((planted < a).sum()), err), flush=True)
        assert err <= TOL[dtype], "window at %d: %.3e" % (a, err)
        if b == L:
            ef = rel_err(fin.cpu().double().numpy(), rfin)
            print("  final_state max|err|/RMS = %.3e" % ef, flush=True)
            assert ef <= TOL[dtype]
    del q, k, v, la, li, out, fin
    torch.cuda.empty_cache()


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
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 192), (256, 64), (100, 64), (96, 80), (48, 16)])
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


# ------------------------------------------------------------------------------ empty calls
def test_empty_calls(gpu_lib):
    # B, H or L of zero: no output rows, and the state after no tokens is the state before
    # them, bit for bit (or zero without one); the backward passes the final-state gradient
    # through to the initial state, and a fixed per-head gate gets a zero gradient
    dev = "cuda"
    g = torch.Generator().manual_seed(5)
    s0 = torch.randn(2, 3, 128, 64, generator=g).to(dev)
    q = torch.zeros(2, 3, 0, 128, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(2, 3, 0, 64, dtype=torch.bfloat16, device=dev)
    for gate, la in (("channel", torch.zeros(2, 3, 0, 128, device=dev)), ("head", torch.zeros(2, 3, 0, device=dev)),
                     ("head_const", torch.full((3,), -0.1, device=dev)), ("none", None)):
        out, fin = gpu_lib.fwd(q, q, v, la, initial_state=s0, chunk=64)
        torch.cuda.synchronize()
        assert out.shape == (2, 3, 0, 64), gate
        assert torch.equal(fin, s0), gate
        out, fin = gpu_lib.fwd(q, q, v, la, chunk=64)
        torch.cuda.synchronize()
        assert torch.count_nonzero(fin).item() == 0, gate
    # no (batch, head) slices
    out, fin = gpu_lib.fwd(q[:0], q[:0], v[:0], None, chunk=64)
    torch.cuda.synchronize()
    assert out.numel() == 0 and fin.numel() == 0
    # delta rule
    beta = torch.zeros(2, 3, 0, device=dev)
    o, fin = gpu_lib.delta_fwd(q, q, v, beta, torch.zeros(2, 3, 0, device=dev), initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 64) and torch.equal(fin, s0)
    # mLSTM: the stabilised state (C', n', m) passes through, or is zero
    n0 = torch.randn(2, 3, 128, generator=g).to(dev)
    m0 = torch.randn(2, 3, generator=g).to(dev)
    lz = torch.zeros(2, 3, 0, device=dev)
    h, (C, n, m) = gpu_lib.mlstm_fwd(q, q, v, lz, lz, initial_state=(s0, n0, m0))
    torch.cuda.synchronize()
    assert h.shape == (2, 3, 0, 64) and torch.equal(C, s0) and torch.equal(n, n0) and torch.equal(m, m0)
    h, (C, n, m) = gpu_lib.mlstm_fwd(q, q, v, lz, lz)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == torch.count_nonzero(n).item() == torch.count_nonzero(m).item() == 0
    # backward
    df = torch.randn(2, 3, 128, 64, generator=g).to(dev)
    la = torch.full((3,), -0.1, device=dev)
    r = gpu_lib.bwd(q, q, v, torch.zeros(2, 3, 0, 64, device=dev), la, initial_state=s0, dfinal_state=df)
    torch.cuda.synchronize()
    assert r["dq"].shape == (2, 3, 0, 128) and r["dv"].shape == (2, 3, 0, 64)
    assert torch.equal(r["dinitial_state"], df)
    assert torch.count_nonzero(r["dlog_alpha"]).item() == 0 and r["dlog_alpha"].shape == (3,)
    # a decode step over no sequences
    st = torch.zeros(0, 3, 128, 64, device=dev)
    o = gpu_lib.step(q[:0, :, 0:0].reshape(0, 3, 128), q[:0, :, 0:0].reshape(0, 3, 128),
                     v[:0, :, 0:0].reshape(0, 3, 64), st, None)
    torch.cuda.synchronize()
    assert o.numel() == 0
