"""The allocation-free forward entry point under HIP graph capture: captured once, replayed
with new input contents copied in between (eager work and synchronisation between the
replays), and every replay compared element by element with an eager call on the same
inputs (the kernels are deterministic, so the results must be identical)."""
import pytest
import torch

from gated_linear_rnn_chunkwise_amd import inputs as gin

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, extra fwd arguments)
    "one_segment": (gin.custom(2, 4, 640, 128, 128, 64, gate="channel"), {}),
    "segments": (gin.custom(1, 2, 4096, 128, 128, 64, gate="head", input_gate=True), {"seg_chunks": 8}),
    "padded_shape": (gin.custom(1, 3, 333, 96, 80, 64, gate="channel"), {}),
    "query_tiles": (gin.custom(1, 2, 1000, 128, 128, 256, gate="head_const"), {"query_tiles": True}),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(gpu_lib, name):
    w, kw = CASES[name]
    dev = "cuda"
    sets = [gin.make_inputs(w, seed=s) for s in range(3)]
    keys = [k for k in ("q", "k", "v", "log_alpha", "log_ig") if sets[0][k] is not None]
    static = {k: sets[0][k].to(dev).clone() for k in keys}
    out = torch.empty(w.B, w.H, w.L, w.Dv, device=dev)
    fin = torch.empty(w.B, w.H, w.Dk, w.Dv, device=dev)

    def call(t, o, f):
        return gpu_lib.fwd_noalloc(t["q"], t["k"], t["v"], t.get("log_alpha"), log_ig=t.get("log_ig"),
                                   chunk=w.chunk, out=o, final_state=f, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static, out, fin)  # warm-up outside the capture (per-device set-up)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(static, out, fin)
    torch.cuda.synchronize()
    for rep in range(5):
        src = sets[rep % 3]
        for k in keys:
            static[k].copy_(src[k].to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out = torch.empty_like(out)
        ref_fin = torch.empty_like(fin)
        eager = {k: src[k].to(dev) for k in keys}
        call(eager, ref_out, ref_fin)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "%s: replay %d output differs from the eager call" % (name, rep)
        assert torch.equal(fin, ref_fin), "%s: replay %d final state differs from the eager call" % (name, rep)
