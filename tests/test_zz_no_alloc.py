"""gla_fwd_noalloc (the forward pass that allocates nothing; its scratch is a fixed device
array per GPU) through the C ABI, against gla_fwd_ex on the same inputs, on two calls in a
row: the second smaller, so it runs on the scratch contents the first left behind.  The
kernels are the same, so the results must agree bit for bit; the oracle bar is checked too."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_linear_rnn_chunkwise_amd import inputs as gin

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}


def rel_err(got, ref):
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def call(gla, entry, w, d, seg_chunks, tile_pairs, s0=None):
    dev = "cuda"
    cu = lambda t: None if t is None else t.to(dev).contiguous()
    q, k, v, la, li, s0g = cu(d["q"]), cu(d["k"]), cu(d["v"]), cu(d["log_alpha"]), cu(d["log_ig"]), cu(s0)
    out = torch.full((w.B, w.H, w.L, w.Dv), float("nan"), device=dev)
    fin = torch.full((w.B, w.H, w.Dk, w.Dv), float("nan"), device=dev)
    desc = gla.make_desc(q, k, v, la, li, s0g, out, fin, w.chunk, seg_chunks, tile_pairs=tile_pairs)
    lib = gla.load()
    st = getattr(lib, entry)(ctypes.byref(desc), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == gla.GLA_OK, (entry, gla.status_string(st))
    return out.cpu().double().numpy(), fin.cpu().double().numpy()


CASES = [
    # (first call, second smaller call): segmented runs (segment-state scratch) and the
    # tile-pair form with a per-channel gate (scaled-key scratch)
    (dict(B=2, H=3, L=3000, Dk=128, Dv=128, chunk=64, gate="channel", seg=4, tp=False),
     dict(B=1, H=2, L=1000, Dk=128, Dv=128, chunk=64, gate="channel", seg=2, tp=False)),
    (dict(B=1, H=4, L=2000, Dk=128, Dv=128, chunk=256, gate="channel", seg=2, tp=True),
     dict(B=1, H=2, L=700, Dk=64, Dv=64, chunk=128, gate="channel", seg=1, tp=True)),
    (dict(B=1, H=2, L=4000, Dk=256, Dv=128, chunk=64, gate="head", ig=True, seg=5, tp=False),
     dict(B=1, H=1, L=900, Dk=256, Dv=64, chunk=64, gate="head", ig=True, seg=3, tp=False)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_general_entry_point(gpu_lib, first, second):
    for i, c in enumerate((first, second)):
        w = gin.custom(c["B"], c["H"], c["L"], c["Dk"], c["Dv"], c["chunk"], gate=c["gate"],
                       input_gate=c.get("ig", False))
        d = gin.make_inputs(w, seed=40 + i)
        s0 = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=torch.Generator().manual_seed(7 + i)) * 0.1
        print("noalloc call %d: %s seg_chunks=%d tile_pairs=%s" % (i, w.name, c["seg"], c["tp"]), flush=True)
        a, fa = call(gpu_lib, "gla_fwd_noalloc", w, d, c["seg"], c["tp"], s0)
        b, fb = call(gpu_lib, "gla_fwd_ex", w, d, c["seg"], c["tp"], s0)
        assert np.array_equal(a, b) and np.array_equal(fa, fb)
        ref, rfin = oracle.recurrent(d["q"], d["k"], d["v"], w.gate, d["log_alpha"], d["log_ig"], s0)
        assert rel_err(a, ref) <= TOL[w.dtype] and rel_err(fa, rfin) <= TOL[w.dtype]


def test_noalloc_without_scratch_and_twice_on_full_workload(gpu_lib):
    # a call that needs no scratch (one segment), then the long-sequence workload twice in a
    # row, whose segment states fill part of the scratch
    w = gin.custom(2, 2, 300, 128, 128, 64, gate="channel")
    d = gin.make_inputs(w, seed=3)
    a, fa = call(gpu_lib, "gla_fwd_noalloc", w, d, 0, False)
    b, fb = call(gpu_lib, "gla_fwd_ex", w, d, 0, False)
    assert np.array_equal(a, b) and np.array_equal(fa, fb)
    w = gin.WORKLOADS["long_gla_bf16_H16L32768_C64"]
    d = gin.make_inputs(w, seed=0)
    b, fb = call(gpu_lib, "gla_fwd_ex", w, d, 0, False)
    for _ in range(2):
        a, fa = call(gpu_lib, "gla_fwd_noalloc", w, d, 0, False)
        assert np.array_equal(a, b) and np.array_equal(fa, fb)
